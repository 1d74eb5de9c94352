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

// A round fused with the layout swap that follows it, for arrays small
// enough for LDS: a row holds N/S arrays of S = A*M*n elements, [A][M][n] in
// the round's layout (fibers of n along the last axis), and each output
// array takes the same place as [n][M][A]. A workgroup takes array p of 32
// consecutive rows: it loads them into LDS (16-byte pieces, row pitch S + 8
// elements), multiplies every fiber in place (wave w takes fibers w, w + 4,
// ...; all of its fibers' weight fragments in registers, requested before
// the arrays; one MFMA per 16 outputs and the lane-quad transpose, as
// fiber_kernel) and writes the arrays out transposed in 16-byte pieces of 8
// consecutive a.
// Input and output arrays cover the same bytes of a row, so `in` may equal
// `out`: a workgroup reads all of its region before it writes any of it.
constexpr int kFsRows = 32;
constexpr int64_t kFsMaxArray = 1024;   // elements: 32 rows of LDS in 66 KB

template <int NN>
__global__ __launch_bounds__(256) void fiber_swap_kernel(const uint16_t* in,
                                                        const uint16_t* __restrict__ w,
                                                        uint16_t* out, int64_t B, int64_t N,
                                                        int S, int A, int M, int npre) {
  extern __shared__ __attribute__((aligned(16))) unsigned char fs_smem[];
  uint16_t* sm = reinterpret_cast<uint16_t*>(fs_smem);
  constexpr int NT = (NN + 15) / 16;
  const int pitch = S + 8;
  const int p = static_cast<int>(blockIdx.x % npre);
  const int64_t r0 = static_cast<int64_t>(blockIdx.x / npre) * kFsRows;
  const int nr = static_cast<int>(B - r0 < kFsRows ? B - r0 : kFsRows);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l15 = lane & 15, lh = lane >> 4;
  const int64_t off = static_cast<int64_t>(p) * S;
  const int pieces = S / 8;
  const int nfib = A * M;
  const bool kin = 8 * lh < NN;   // this lane's k are real

  // weight fragments of this wave's fibers w + 4i, requested before the
  // arrays so that both are in flight together
  constexpr int FMAX = static_cast<int>((kFsMaxArray / NN + 3) / 4);
  u32x4 bv[FMAX][NT];
#pragma unroll
  for (int i = 0; i < FMAX; ++i) {
    const int f = wv + 4 * i;
    const int64_t gf = static_cast<int64_t>(p) * nfib + f;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int pr = 16 * j + l15;
      bv[i][j] = f < nfib && kin && pr < NN
                     ? *reinterpret_cast<const u32x4*>(w + (gf * NN + pr) * NN + 8 * lh)
                     : u32x4{0u, 0u, 0u, 0u};
    }
  }

  // rows past the batch read the last row (never stored)
  for (int q = tid; q < kFsRows * pieces; q += 256) {
    const int r = q / pieces, pc = q - r * pieces;
    const int64_t row = r0 + (r < nr ? r : nr - 1);
    *reinterpret_cast<u32x4*>(sm + r * pitch + pc * 8) =
        *reinterpret_cast<const u32x4*>(in + row * N + off + pc * 8);
  }
  __syncthreads();

#pragma unroll
  for (int i = 0; i < FMAX; ++i) {
    const int f = wv + 4 * i;
    if (f >= nfib) break;
#pragma unroll
    for (int rg = 0; rg < kFsRows / 16; ++rg) {
      uint16_t* base = sm + (16 * rg) * pitch + f * NN;
      const u32x4 av = kin ? *reinterpret_cast<const u32x4*>(base + l15 * pitch + 8 * lh)
                           : u32x4{0u, 0u, 0u, 0u};
      f32x4 o[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j)
        o[j] = quad_transpose4(__builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                   as_op(av), as_op(bv[i][j]), f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0),
                               lane & 3);
      // the fiber's inputs were read (above) before its outputs overwrite
      // them; other waves own other fibers
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int p0 = 16 * j + (l15 & ~3);
        if (p0 < NN)
          *reinterpret_cast<u32x2*>(base + (4 * lh + (lane & 3)) * pitch + p0) =
              u32x2{pack_bf16x2(o[j][0], o[j][1]), pack_bf16x2(o[j][2], o[j][3])};
      }
    }
  }
  __syncthreads();

  // two output pieces per pass: 8 consecutive a of (c, m) and of (c + 1, m),
  // from 4-byte LDS reads of the element pairs (c, c + 1) of each a (c even)
  const int na8 = A / 8, dpr = S / 16;
  for (int q = tid; q < nr * dpr; q += 256) {
    const int r = q / dpr, dp = q - r * dpr;
    const int a0 = (dp % na8) * 8, rest = dp / na8, m = rest % M, c = 2 * (rest / M);
    const uint32_t* src =
        reinterpret_cast<const uint32_t*>(sm + r * pitch + (a0 * M + m) * NN + c);
    uint32_t x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = src[e * M * NN / 2];
    u32x4 lo, hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo[e] = (x[2 * e] & 0xffffu) | (x[2 * e + 1] << 16);
      hi[e] = (x[2 * e] >> 16) | (x[2 * e + 1] & 0xffff0000u);
    }
    uint16_t* dst = out + (r0 + r) * N + off + a0;
    *reinterpret_cast<u32x4*>(dst + (c * M + m) * A) = lo;
    *reinterpret_cast<u32x4*>(dst + ((c + 1) * M + m) * A) = hi;
  }
}

// Round 0 of a lattice joined with the transposes between the natural
// layout and L_0 (axis 0 last): fiber f of axis 0 (f < R = N/n, the index of
// the other axes) has its n elements at c*R + f in the natural layout and at
// f*n + c in L_0. A workgroup takes 16 rows and 64 consecutive fibers (fewer
// in a last chunk, a multiple of 8), held in LDS as [row][fiber][n] (row
// pitch 64n + 8 elements). Forward (DIR 0): x is read in 16-byte pieces of 8
// consecutive fibers of one element, 8 pieces per task (128-byte runs across
// the tasks of a wave), and turned by 8x8 register transposes into LDS; the
// L_0 copy of x (the weight gradient's input) is written, the fibers are
// multiplied in place (wave w: fibers 16w .. 16w + 15, weights preloaded;
// one MFMA per 16 outputs and the lane-quad transpose) and the results are
// written in L_0. Backward (DIR 1): the gradient in L_0 is read straight
// into LDS, multiplied with the per-fiber transposed weights, and written to
// dx in the natural layout through the same transposes.
constexpr int kStRows = 16, kStFib = 64;

template <int NN, int DIR>
__global__ __launch_bounds__(256) void fiber_strided_kernel(const uint16_t* __restrict__ in,
                                                           const uint16_t* __restrict__ w,
                                                           uint16_t* __restrict__ out,
                                                           uint16_t* __restrict__ save, int64_t B,
                                                           int64_t N, int nchunks) {
  extern __shared__ __attribute__((aligned(16))) unsigned char st_smem[];
  uint16_t* sm = reinterpret_cast<uint16_t*>(st_smem);
  constexpr int NT = (NN + 15) / 16;
  constexpr int PITCH = kStFib * NN + 8;
  constexpr int FW = kStFib / 4;   // fibers per wave
  constexpr int NG = NN / 8;       // 8-element groups of a fiber
  const int64_t R = N / NN;
  const int fc = static_cast<int>(blockIdx.x % nchunks);
  const int64_t r0 = static_cast<int64_t>(blockIdx.x / nchunks) * kStRows;
  const int nr = static_cast<int>(B - r0 < kStRows ? B - r0 : kStRows);
  const int64_t f0 = static_cast<int64_t>(fc) * kStFib;
  const int nfb = static_cast<int>(R - f0 < kStFib ? R - f0 : kStFib);
  const int nf8 = nfb / 8;
  const int per = nfb * NG;        // 16-byte pieces of a row's chunk in L_0
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l15 = lane & 15, lh = lane >> 4;
  const bool kin = 8 * lh < NN;

  u32x4 bv[FW][NT];
#pragma unroll
  for (int i = 0; i < FW; ++i) {
    const int f = FW * wv + i;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int pr = 16 * j + l15;
      bv[i][j] = f < nfb && kin && pr < NN
                     ? *reinterpret_cast<const u32x4*>(w + ((f0 + f) * NN + pr) * NN + 8 * lh)
                     : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // rows past the batch read the last row (never stored)
  auto copy_out = [&](uint16_t* dst) {
    for (int q = tid; q < nr * per; q += 256) {
      const int r = q / per, pc = q - r * per;
      *reinterpret_cast<u32x4*>(dst + (r0 + r) * N + f0 * NN + pc * 8) =
          *reinterpret_cast<const u32x4*>(sm + r * PITCH + pc * 8);
    }
  };
  if constexpr (DIR == 0) {
    // task (row r, element group cg, fiber group fg), fg fastest
    for (int t = tid; t < kStRows * NG * nf8; t += 256) {
      const int fg = t % nf8, rest = t / nf8, cg = rest % NG, r = rest / NG;
      const int64_t row = r0 + (r < nr ? r : nr - 1);
      const uint16_t* src = in + row * N + static_cast<int64_t>(cg * 8) * R + f0 + fg * 8;
      u32x4 v[8], tr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const u32x4*>(src + i * R);
      transpose8x8(v, tr);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<u32x4*>(sm + r * PITCH + (fg * 8 + e) * NN + cg * 8) = tr[e];
    }
    __syncthreads();
    copy_out(save);
    __syncthreads();
  } else {
    for (int q = tid; q < kStRows * per; q += 256) {
      const int r = q / per, pc = q - r * per;
      const int64_t row = r0 + (r < nr ? r : nr - 1);
      *reinterpret_cast<u32x4*>(sm + r * PITCH + pc * 8) =
          *reinterpret_cast<const u32x4*>(in + row * N + f0 * NN + pc * 8);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < FW; ++i) {
    const int f = FW * wv + i;
    if (f >= nfb) break;
    uint16_t* base = sm + f * NN;
    const u32x4 av = kin ? *reinterpret_cast<const u32x4*>(base + l15 * PITCH + 8 * lh)
                         : u32x4{0u, 0u, 0u, 0u};
    f32x4 o[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j)
      o[j] = quad_transpose4(__builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                 as_op(av), as_op(bv[i][j]), f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0),
                             lane & 3);
    // the fiber's inputs were read (above) before its outputs overwrite them
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int p0 = 16 * j + (l15 & ~3);
      if (p0 < NN)
        *reinterpret_cast<u32x2*>(base + (4 * lh + (lane & 3)) * PITCH + p0) =
            u32x2{pack_bf16x2(o[j][0], o[j][1]), pack_bf16x2(o[j][2], o[j][3])};
    }
  }
  __syncthreads();
  if constexpr (DIR == 0) {
    copy_out(out);
  } else {
    // task (row r, output group pg, fiber group fg): outputs pg*8 + i of
    // fibers fg*8 .. fg*8 + 7 -> dx[row, (pg*8 + i)*R + f0 + fg*8 ..]
    for (int t = tid; t < nr * NG * nf8; t += 256) {
      const int fg = t % nf8, rest = t / nf8, pg = rest % NG, r = rest / NG;
      u32x4 v[8], tr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[e] = *reinterpret_cast<const u32x4*>(sm + r * PITCH + (fg * 8 + e) * NN + pg * 8);
      transpose8x8(v, tr);
      uint16_t* dst = out + (r0 + r) * N + static_cast<int64_t>(pg * 8) * R + f0 + fg * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(dst + i * R) = tr[i];
    }
  }
}

}  // namespace

bool fiber_applicable(int64_t n, bool bf16) { return bf16 && (n == 16 || n == 24 || n == 32); }

bool fiber_strided_applicable(int64_t n, int64_t N, bool bf16) {
  return fiber_applicable(n, bf16) && N % n == 0 && (N / n) % 8 == 0;
}

hipError_t launch_fiber_strided(const void* in, const void* w, void* out, void* save,
                                int64_t batch, int64_t N, int64_t n, int dir, bool bf16,
                                hipStream_t s) {
  if (!fiber_strided_applicable(n, N, bf16) || (dir == 0 && !save)) return hipErrorInvalidValue;
  if (batch <= 0) return hipSuccess;
  const int64_t R = N / n, nchunks = (R + kStFib - 1) / kStFib;
  const int64_t grid = nchunks * ((batch + kStRows - 1) / kStRows);
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const size_t lds = static_cast<size_t>(kStRows) * (kStFib * n + 8) * 2;
  const uint16_t* ip = static_cast<const uint16_t*>(in);
  const uint16_t* wp = static_cast<const uint16_t*>(w);
  uint16_t* op = static_cast<uint16_t*>(out);
  uint16_t* sp = static_cast<uint16_t*>(save);
  const dim3 gd(static_cast<unsigned>(grid));
  const int nc = static_cast<int>(nchunks);
#define MONARCH_STRIDED(NN)                                                                     \
  if (dir == 0)                                                                                 \
    hipLaunchKernelGGL((fiber_strided_kernel<NN, 0>), gd, dim3(256), lds, s, ip, wp, op, sp,    \
                       batch, N, nc);                                                           \
  else                                                                                          \
    hipLaunchKernelGGL((fiber_strided_kernel<NN, 1>), gd, dim3(256), lds, s, ip, wp, op, sp,    \
                       batch, N, nc)
  switch (n) {
    case 16: MONARCH_STRIDED(16); break;
    case 24: MONARCH_STRIDED(24); break;
    default: MONARCH_STRIDED(32); break;
  }
#undef MONARCH_STRIDED
  return hipGetLastError();
}

bool fiber_swap_applicable(int64_t n, int64_t A, int64_t M, bool bf16) {
  return fiber_applicable(n, bf16) && A > 0 && M > 0 && A % 8 == 0 && A * M * n <= kFsMaxArray;
}

hipError_t launch_fiber_swap(const void* in, const void* w, void* out, int64_t batch, int64_t N,
                             int64_t n, int64_t A, int64_t M, bool bf16, hipStream_t s) {
  const int64_t S = A * M * n;
  if (!fiber_swap_applicable(n, A, M, bf16) || N % S) return hipErrorInvalidValue;
  if (batch <= 0) return hipSuccess;
  const int64_t npre = N / S;
  const int64_t grid = npre * ((batch + kFsRows - 1) / kFsRows);
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const size_t lds = static_cast<size_t>(kFsRows) * (S + 8) * 2;
  const uint16_t* ip = static_cast<const uint16_t*>(in);
  const uint16_t* wp = static_cast<const uint16_t*>(w);
  uint16_t* op = static_cast<uint16_t*>(out);
  const dim3 gd(static_cast<unsigned>(grid));
  const int Si = static_cast<int>(S), Ai = static_cast<int>(A), Mi = static_cast<int>(M),
            Pi = static_cast<int>(npre);
  switch (n) {
    case 16: hipLaunchKernelGGL(fiber_swap_kernel<16>, gd, dim3(256), lds, s, ip, wp, op, batch, N, Si, Ai, Mi, Pi); break;
    case 24: hipLaunchKernelGGL(fiber_swap_kernel<24>, gd, dim3(256), lds, s, ip, wp, op, batch, N, Si, Ai, Mi, Pi); break;
    default: hipLaunchKernelGGL(fiber_swap_kernel<32>, gd, dim3(256), lds, s, ip, wp, op, batch, N, Si, Ai, Mi, Pi); break;
  }
  return hipGetLastError();
}

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
