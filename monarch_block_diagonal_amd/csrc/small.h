// Launchers of the fused 32x32-block bf16 path (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace monarch {

// True when the fused path covers the problem: bf16, in = out = 32*nb with
// nb1 = nb2 = nb, nb in {8, 16, 32}, batch >= 1 and batch*out < 2^31.
bool sm_applicable(int64_t in, int64_t out, int64_t nb1, int64_t nb2, int64_t batch,
                   int dtype_bf16);

// Forward: y and z (row-major W[b, g*32 + t] = Z[b, t*nb + g], the generic
// path's stage-2-order z) from x.
hipError_t sm_launch_fwd(const void* x, const void* w1, const void* w2, void* y, void* z,
                         int64_t batch, int64_t nb, int relu, hipStream_t s);
// Backward data: dx, and dv (row-major dV[b, g*32 + p]) and dz (row-major
// Z order) for the weight gradients; ymask (y of the forward, or NULL) masks
// dy by y > 0.
hipError_t sm_launch_bwd_data(const void* dy, const void* ymask, const void* w1, const void* w2,
                              void* dx, void* dv, void* dz, int64_t batch, int64_t nb,
                              hipStream_t s);

// Batch split of the weight gradients (chunks of >= 256 rows, <= 64 chunks).
void sm_wgrad_split(int64_t batch, int64_t* splits, int64_t* chunk);
// Both weight gradients as fp32 partials [splits][nb][32][32]: part_l from
// dv and z (row-major W order), part_r from dz (Z order) and x.
hipError_t sm_launch_wgrad(const void* dv, const void* z, const void* dz, const void* x,
                           float* part_l, float* part_r, int64_t batch, int64_t nb,
                           hipStream_t s);

}  // namespace monarch
