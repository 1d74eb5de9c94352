// Launchers of the 128x128-block bf16 fast path (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace monarch {

// Launch geometry of the fast path for one batch size.
struct SqPlan {
  int64_t fwd1_chunks = 0, fwd1_rows = 0;  // stage-1 forward: row chunks per block
  int64_t s2_ranges = 0, s2_rows = 0;      // stage-2 forward: row ranges per block group
  int64_t d2_ranges = 0, d2_rows = 0;      // stage-2 backward data: row ranges per group
  int64_t w2_chunks = 0, w2_rows = 0;      // stage-2 weight gradient: batch chunks
  int64_t b1_chunks = 0, b1_rows = 0;      // stage-1 backward: batch chunks
};

// True when the fast path covers the problem: bf16, in = out = 128*nb with
// nb1 = nb2 = nb, nb in {32, 64, 128}, and batch*out < 2^31.
bool sq_applicable(int64_t in, int64_t out, int64_t nb1, int64_t nb2, int64_t batch,
                   int dtype_bf16);
SqPlan sq_plan(int64_t batch, int64_t nb);

// Tile-major panel layout (F features per row): feature f of row b at
// (b - b%16)*F + ((f/8)*rt + b%16)*8 + f%8, rt = rows of b's 16-row tile
// (16, or batch%16 in a last partial tile). z holds
// stage 2's input W[b, g*128 + t] = Z[b, t*nb + g] in it; dz holds dZ (Z order).
hipError_t sq_launch_stage1_fwd(const void* x, const void* w1, void* z, int64_t batch, int64_t nb,
                                const SqPlan& p, hipStream_t s);
hipError_t sq_launch_stage2_fwd(const void* z, const void* w2, void* y, int64_t batch, int64_t nb,
                                int relu, const SqPlan& p, hipStream_t s);
// dv = dY (masked by ymask > 0 when ymask is set) in block-major panels:
// feature g*128 + p of row b in the panel layout.
hipError_t sq_launch_dv_panels(const void* dy, const void* ymask, void* dv, int64_t batch,
                               int64_t nb, hipStream_t s);
hipError_t sq_launch_stage2_bwd_data(const void* dv, const void* w2, void* dz, int64_t batch,
                                     int64_t nb, const SqPlan& p, hipStream_t s);
// partial: [w2_chunks][nb][128][128] fp32
hipError_t sq_launch_stage2_bwd_weight(const void* dv, const void* z, float* partial,
                                       int64_t batch, int64_t nb, const SqPlan& p, hipStream_t s);
// partial: [b1_chunks][nb][128][128] fp32
hipError_t sq_launch_stage1_bwd(const void* dz, const void* x, const void* w1, void* dx,
                                float* partial, int64_t batch, int64_t nb, const SqPlan& p,
                                hipStream_t s);

}  // namespace monarch
