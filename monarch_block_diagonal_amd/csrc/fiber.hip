// Rounds of the k-factor ("hypercube") layer on short fibers (scatterbrain
// issues page, "hypercube" thread: round j multiplies every fiber of axis j
// by its own n_j x n_j matrix): bf16, n in {16, 24, 32}.
//
//   out[b, f*n + p] = sum_t M[f][p][t] in[b, f*n + t]
//
// with M the round's weights (forward) or their per-fiber transposes (data
// gradient). A fiber's whole contraction is one v_mfma_f32_16x16x32_bf16 per
// 16 outputs (K = n <= 32, the k past n zeroed), so the work is the data
// movement. Each wave owns 16 rows and a segment of F = 256/n consecutive
// fibers: it reads the segment (a run of up to 512 bytes per row) with
// 16-byte loads into its own LDS rows, and all of the segment's 16-byte
// weight fragments into registers at the same time (they come from cache:
// every row tile of the launch reads the same weights); it then multiplies
// fiber by fiber (A fragments from LDS), writes each fiber's results
// back over its inputs after a 4 x 4 transpose within lane quads, and
// stores the segment with 16-byte stores. Waves share nothing, so no barrier
// is needed. Workgroup: 4 waves (64 rows) on one segment.
#include "common.h"
#include "kernels.h"

namespace monarch {
namespace {

__device__ __forceinline__ bf16x8 as_op(u32x4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
}

// 4x4 transpose within lane quads: lane 4c+u holds column 4c+u of rows
// 4*lh + (0..3) in `in`; returns row 4*lh + u, columns 4c..4c+3.
__device__ __forceinline__ f32x4 quad_transpose(f32x4 in, int lane) {
  const int u = lane & 3;
  f32x4 o;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int sr = (u - r) & 3;
    const float send = sr == 0 ? in[0] : sr == 1 ? in[1] : sr == 2 ? in[2] : in[3];
    const float got = __shfl(send, (lane & ~3) | ((u + r) & 3), 64);
    const int dc = (u + r) & 3;
    o[0] = dc == 0 ? got : o[0];
    o[1] = dc == 1 ? got : o[1];
    o[2] = dc == 2 ? got : o[2];
    o[3] = dc == 3 ? got : o[3];
  }
  return o;
}

constexpr int kSeg = 256;          // elements of a fiber segment (at most)
constexpr int kSegPitch = kSeg + 8;

template <int NN>   // fiber length
__global__ __launch_bounds__(256) void fiber_kernel(const uint16_t* __restrict__ in,
                                                   const uint16_t* __restrict__ w,
                                                   uint16_t* __restrict__ out, int64_t B,
                                                   int64_t N, int64_t segs) {
  constexpr int F = kSeg / NN;               // fibers per segment
  constexpr int NT = (NN + 15) / 16;         // 16-wide output tiles per fiber
  __shared__ __attribute__((aligned(16))) uint16_t ls[4][16 * kSegPitch];
  const int64_t nf = N / NN;
  const int64_t sg = blockIdx.x % segs;
  const int64_t b0 = static_cast<int64_t>(blockIdx.x / segs) * 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l15 = lane & 15, lh = lane >> 4;
  uint16_t* s = ls[wv];
  const int64_t rbase = b0 + 16 * wv;
  const int64_t f0 = sg * F;
  const int nfs = static_cast<int>(f0 + F < nf ? F : nf - f0);   // fibers here
  const int ppr = nfs * NN / 8;                                 // 16-byte pieces per row
  const int64_t col0 = f0 * NN;
  const bool kin = 8 * lh < NN;                                 // this lane's k are real

  // weight fragments of the segment: W[f][p = 16j + l15][t = 8lh ..]
  u32x4 bv[F][NT];
#pragma unroll
  for (int fl = 0; fl < F; ++fl)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int p = 16 * j + l15;
      bv[fl][j] = kin && p < NN && fl < nfs
                      ? *reinterpret_cast<const u32x4*>(w + ((f0 + fl) * NN + p) * NN + 8 * lh)
                      : u32x4{0u, 0u, 0u, 0u};
    }
  // segment rows -> LDS (rows past the batch read the last row; never stored)
  for (int idx = lane; idx < 16 * ppr; idx += 64) {
    const int r = idx / ppr, pc = idx - r * ppr;
    const int64_t row = rbase + r < B ? rbase + r : B - 1;
    *reinterpret_cast<u32x4*>(s + r * kSegPitch + pc * 8) =
        *reinterpret_cast<const u32x4*>(in + row * N + col0 + pc * 8);
  }
#pragma unroll
  for (int fl = 0; fl < F; ++fl) {
    if (fl < nfs) {
      const u32x4 av = kin ? *reinterpret_cast<const u32x4*>(s + l15 * kSegPitch + fl * NN + 8 * lh)
                           : u32x4{0u, 0u, 0u, 0u};
      f32x4 o[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j)
        o[j] = quad_transpose(__builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                  as_op(av), as_op(bv[fl][j]), f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0),
                              lane);
      // every lane has read this fiber's inputs (one instruction above)
      // before any lane writes its outputs over them
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int p0 = 16 * j + (l15 & ~3);
        if (p0 < NN)
          *reinterpret_cast<u32x2*>(s + (4 * lh + (lane & 3)) * kSegPitch + fl * NN + p0) =
              u32x2{pack_bf16x2(o[j][0], o[j][1]), pack_bf16x2(o[j][2], o[j][3])};
      }
    }
  }
  for (int idx = lane; idx < 16 * ppr; idx += 64) {
    const int r = idx / ppr, pc = idx - r * ppr;
    if (rbase + r < B)
      *reinterpret_cast<u32x4*>(out + (rbase + r) * N + col0 + pc * 8) =
          *reinterpret_cast<const u32x4*>(s + r * kSegPitch + pc * 8);
  }
}

}  // namespace

bool fiber_applicable(int64_t n, bool bf16) { return bf16 && (n == 16 || n == 24 || n == 32); }

hipError_t launch_fiber(const void* in, const void* w, void* out, int64_t batch, int64_t N,
                        int64_t n, bool bf16, hipStream_t s) {
  if (!fiber_applicable(n, bf16) || N % n) return hipErrorInvalidValue;
  if (batch <= 0) return hipSuccess;
  const int64_t per = kSeg / n;
  const int64_t segs = (N / n + per - 1) / per;
  const int64_t grid = segs * ((batch + 63) / 64);
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const uint16_t* ip = static_cast<const uint16_t*>(in);
  const uint16_t* wp = static_cast<const uint16_t*>(w);
  uint16_t* op = static_cast<uint16_t*>(out);
  const dim3 g(static_cast<unsigned>(grid));
  switch (n) {
    case 16: hipLaunchKernelGGL(fiber_kernel<16>, g, dim3(256), 0, s, ip, wp, op, batch, N, segs); break;
    case 24: hipLaunchKernelGGL(fiber_kernel<24>, g, dim3(256), 0, s, ip, wp, op, batch, N, segs); break;
    default: hipLaunchKernelGGL(fiber_kernel<32>, g, dim3(256), 0, s, ip, wp, op, batch, N, segs); break;
  }
  return hipGetLastError();
}

}  // namespace monarch
