// Rounds of the k-factor ("hypercube") layer on short fibers (scatterbrain
// issues page, "hypercube" thread: round j multiplies every fiber of axis j
// by its own n_j x n_j matrix): bf16, n in {16, 24, 32}.
//
//   out[b, f*n + p] = sum_t M[f][p][t] in[b, f*n + t]
//
// with M the round's weights (forward) or their per-fiber transposes (data
// gradient). A fiber's whole contraction is one v_mfma_f32_16x16x32_bf16 per
// 16 outputs (K = n <= 32, the k past n zeroed), so the work is the data
// movement. Each wave owns 16 rows and a segment of F consecutive fibers
// (256/n, or 8 for n = 24: a run of 512 or 384 bytes per row, starting on a
// 128-byte line): it reads the segment with
// 16-byte loads into its own LDS rows, and all of the segment's 16-byte
// weight fragments into registers at the same time (they come from cache:
// every row tile of the launch reads the same weights); it then multiplies
// fiber by fiber (A fragments from LDS), writes each fiber's results
// back over its inputs after a 4 x 4 transpose within lane quads, and
// stores the segment with 16-byte stores. Waves share nothing, so no barrier
// is needed. Workgroup: 4 waves (64 rows) on one segment.
//
// The weight gradient of a round, dW[f][p][t] = sum_b G[b, f*n + p]
// I[b, f*n + t] (G: gradient of the round's output, I: its input), runs per
// segment and batch chunk: 32-row steps of both operands are read as 16-byte
// pieces (the same segments), transposed in registers (4 rows x 8
// features per thread) into [feature][row] LDS tiles, and each wave sums whole
// fibers' n x n gradients with MFMAs of K = 32 rows; one fp32 partial per
// chunk, reduced in a fixed order afterwards.
#include "common.h"
#include "kernels.h"

namespace monarch {
namespace {

__device__ __forceinline__ bf16x8 as_op(u32x4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
}

constexpr int kSeg = 256;          // elements of a fiber segment (at most)
constexpr int kSegPitch = kSeg + 8;

// fibers per segment: 256 elements for n = 16 and 32; 8 fibers (192
// elements, three 128-byte lines of bf16) for n = 24, so that segments start
// on cache-line boundaries
__host__ __device__ constexpr int seg_fibers(int n) { return n == 24 ? 8 : kSeg / n; }

template <int NN>   // fiber length
__global__ __launch_bounds__(256) void fiber_kernel(const uint16_t* __restrict__ in,
                                                   const uint16_t* __restrict__ w,
                                                   uint16_t* __restrict__ out, int64_t B,
                                                   int64_t N, int64_t segs) {
  constexpr int F = seg_fibers(NN);          // fibers per segment
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
        o[j] = quad_transpose4(__builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                   as_op(av), as_op(bv[fl][j]), f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0),
                               lane & 3);
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

constexpr int kWKT = 32;            // rows per weight-gradient step
constexpr int kWTP = kWKT + 8;      // LDS pitch of [feature][32 positions]

template <int NN>
__global__ __launch_bounds__(256) void fiber_wgrad_kernel(const uint16_t* __restrict__ G,
                                                         const uint16_t* __restrict__ I,
                                                         float* __restrict__ partial, int64_t B,
                                                         int64_t N, int64_t segs, int64_t chunk) {
  constexpr int F = seg_fibers(NN);            // fibers per segment
  constexpr int NT = (NN + 15) / 16;           // 16-wide tiles per fiber side
  constexpr int FW = (F + 3) / 4;              // fibers per wave (at most)
  __shared__ __attribute__((aligned(16))) uint16_t ts[2][kSeg * kWTP];   // G, I: [feature][pos]
  const int64_t nf = N / NN;
  const int64_t sg = blockIdx.x % segs;
  const int64_t c = blockIdx.x / segs;
  const int64_t r0 = c * chunk;
  const int64_t r1 = r0 + chunk < B ? r0 + chunk : B;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l15 = lane & 15, lh = lane >> 4;
  const int64_t f0 = sg * F;
  const int nfs = static_cast<int>(f0 + F < nf ? F : nf - f0);
  const int ppr = nfs * NN / 8;                // 16-byte pieces per row of the segment
  const int64_t col0 = f0 * NN;

  // loader units u = tid + 256*j (j = 0, 1): operand u / 256 (0: G, 1: I),
  // piece pc = (u / 8) % 32, rows rq + 8i of the step (rq = u % 8); position
  // 4rq + i of a [feature][pos] tile holds row rq + 8i in both operands
  f32x4 acc[FW][NT][NT];
#pragma unroll
  for (int a = 0; a < FW; ++a)
#pragma unroll
    for (int mi = 0; mi < NT; ++mi)
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) acc[a][mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t b0 = r0; b0 < r1; b0 += kWKT) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int u = tid + 256 * j;
      const int op = u >> 8, pc = (u >> 3) & 31, rq = u & 7;
      if (pc < ppr) {
        const uint16_t* src = (op ? I : G) + col0 + pc * 8;
        u32x4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t row = b0 + rq + 8 * i;
          v[i] = row < r1 ? *reinterpret_cast<const u32x4*>(src + row * N) : u32x4{0u, 0u, 0u, 0u};
        }
        u32x2 tr[8];
        transpose4x8(v, tr);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *reinterpret_cast<u32x2*>(&ts[op][(pc * 8 + e) * kWTP + 4 * rq]) = tr[e];
      }
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < FW; ++a) {
      const int fl = wv + 4 * a;
      if (fl < nfs) {
        bf16x8 fa[NT], fb[NT];
#pragma unroll
        for (int mi = 0; mi < NT; ++mi) {
          const int p = 16 * mi + l15;
          fa[mi] = p < NN ? as_op(*reinterpret_cast<const u32x4*>(&ts[0][(fl * NN + p) * kWTP + 8 * lh]))
                          : as_op(u32x4{0u, 0u, 0u, 0u});
        }
#pragma unroll
        for (int ni = 0; ni < NT; ++ni) {
          const int t = 16 * ni + l15;
          fb[ni] = t < NN ? as_op(*reinterpret_cast<const u32x4*>(&ts[1][(fl * NN + t) * kWTP + 8 * lh]))
                          : as_op(u32x4{0u, 0u, 0u, 0u});
        }
#pragma unroll
        for (int mi = 0; mi < NT; ++mi)
#pragma unroll
          for (int ni = 0; ni < NT; ++ni)
            acc[a][mi][ni] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[mi], fb[ni], acc[a][mi][ni], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // partial[c][f][p][t]
#pragma unroll
  for (int a = 0; a < FW; ++a) {
    const int fl = wv + 4 * a;
    if (fl < nfs) {
      float* P = partial + (c * nf + f0 + fl) * NN * NN;
#pragma unroll
      for (int mi = 0; mi < NT; ++mi)
#pragma unroll
        for (int ni = 0; ni < NT; ++ni)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int p = 16 * mi + 4 * lh + v, t = 16 * ni + l15;
            if (p < NN && t < NN) P[p * NN + t] = acc[a][mi][ni][v];
          }
    }
  }
}

}  // namespace

bool fiber_applicable(int64_t n, bool bf16) { return bf16 && (n == 16 || n == 24 || n == 32); }

hipError_t launch_fiber(const void* in, const void* w, void* out, int64_t batch, int64_t N,
                        int64_t n, bool bf16, hipStream_t s) {
  if (!fiber_applicable(n, bf16) || N % n) return hipErrorInvalidValue;
  if (batch <= 0) return hipSuccess;
  const int64_t per = seg_fibers(static_cast<int>(n));
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

void fiber_wgrad_split(int64_t batch, int64_t N, int64_t n, int64_t* splits, int64_t* chunk) {
  // about four workgroups per CU in all, chunks of at least 256 rows
  // (multiples of the 32-row step)
  const int64_t per = seg_fibers(static_cast<int>(n)), segs = (N / n + per - 1) / per;
  int64_t s = (1024 + segs - 1) / segs;
  const int64_t smax = (batch + 255) / 256;
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  int64_t c = (batch + s - 1) / s;
  c = (c + kWKT - 1) / kWKT * kWKT;
  *chunk = c;
  *splits = (batch + c - 1) / c;
}

hipError_t launch_fiber_wgrad(const void* g, const void* in, float* partial, int64_t batch,
                              int64_t N, int64_t n, int64_t chunk, bool bf16, hipStream_t s) {
  if (!fiber_applicable(n, bf16) || N % n || chunk <= 0 || chunk % kWKT) return hipErrorInvalidValue;
  if (batch <= 0) return hipSuccess;
  const int64_t per = seg_fibers(static_cast<int>(n)), segs = (N / n + per - 1) / per;
  const int64_t grid = segs * ((batch + chunk - 1) / chunk);
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const uint16_t* gp = static_cast<const uint16_t*>(g);
  const uint16_t* ip = static_cast<const uint16_t*>(in);
  const dim3 gd(static_cast<unsigned>(grid));
  switch (n) {
    case 16: hipLaunchKernelGGL(fiber_wgrad_kernel<16>, gd, dim3(256), 0, s, gp, ip, partial, batch, N, segs, chunk); break;
    case 24: hipLaunchKernelGGL(fiber_wgrad_kernel<24>, gd, dim3(256), 0, s, gp, ip, partial, batch, N, segs, chunk); break;
    default: hipLaunchKernelGGL(fiber_wgrad_kernel<32>, gd, dim3(256), 0, s, gp, ip, partial, batch, N, segs, chunk); break;
  }
  return hipGetLastError();
}

}  // namespace monarch
