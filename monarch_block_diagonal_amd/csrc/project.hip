// Dense -> Monarch projection (Definition C.3 case, out = nblocks1 * nblocks2).
//
// The scatterbrain issues page ("projection" thread) rearranges M as
// '(p k) (r s) -> k r p s' and fits every (k, r) slice on its own; the
// Monarch paper's abstract calls the result an analytical optimal solution.
// With w1 = R [b1, b2, q1i] and w2 = L [b2, q2o, b1], slice (g, r) over (p, s)
// is A[p][s] = M[p*b2 + g][r*q1i + s] and the Monarch matrix holds
// L[g, p, r] * R[r, g, s] there, so the nearest Monarch matrix takes each
// slice's nearest rank-one matrix sigma * u * vᵀ (top singular triple).
//
// One workgroup per slice: the slice is read once from HBM into LDS (fp32),
// then a fixed number of power iterations v <- normalize(Aᵀ (A v)) run in
// LDS, starting from the column sums of A. The result is split evenly,
// L[g, :, r] = u * sqrt(sigma) (u = A v / sigma), R[r, g, :] = v * sqrt(sigma),
// with the sign chosen so that R's entry of largest magnitude (the first one
// on ties) is positive. Power iteration converges to the top pair at the rate
// (sigma2 / sigma1)^2 per iteration; an exactly rank-one slice is fitted
// after one iteration.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace monarch {
namespace {

constexpr int PT = 256;   // threads per workgroup

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// sum over the workgroup, returned to every thread (red: 8 floats of LDS)
__device__ float block_sum(float x, float* red) {
  x = wave_sum(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < PT / 64; ++i) s += red[i];
  return s;
}

// y[i] = sum_j A(i, j) x[j] for n rows of length len; A(i, j) = base[i*si + j*sj].
// A group of `tpr` adjacent lanes (a power of two <= 64) shares one row.
__device__ void matvec(const float* base, int si, int sj, int n, int len, const float* x,
                       float* y, int tpr) {
  const int part = threadIdx.x & (tpr - 1);
  const int rows_per_pass = PT / tpr;
  for (int i0 = 0; i0 < n; i0 += rows_per_pass) {
    const int i = i0 + static_cast<int>(threadIdx.x) / tpr;
    float acc = 0.f;
    if (i < n)
      for (int j = part; j < len; j += tpr) acc += base[i * si + j * sj] * x[j];
    for (int o = tpr >> 1; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (i < n && part == 0) y[i] = acc;
  }
}

// Sum over the 16 lanes of a DPP row, returned to each of them: swaps within
// quads (lane ^ 1, lane ^ 2), then the two quads of each half (row_half_mirror)
// and the two halves (row_mirror). VALU data movement, no LDS round trip.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL,
                                                            0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);   // row_half_mirror
  x += dpp_mov<0x140>(x);   // row_mirror
  return x;
}

__device__ __forceinline__ int lanes_per_row(int n) {
  int t = 1;
  while (t < 64 && t * 2 * n <= PT) t *= 2;
  return t;
}

template <typename T>
__global__ __launch_bounds__(PT) void project_slices_kernel(const T* __restrict__ M,
                                                            T* __restrict__ W1,
                                                            T* __restrict__ W2, int64_t in,
                                                            int b1, int b2, int q1i, int q2o,
                                                            int iters) {
  extern __shared__ float sm[];
  const int pitch = q1i + 1;             // odd pitch: column walks hit distinct banks
  float* A = sm;                         // [q2o][pitch]
  float* v = A + q2o * pitch;            // [q1i]
  float* u = v + q1i;                    // [q2o]
  float* red = u + q2o;                  // 8 floats
  int* ired = reinterpret_cast<int*>(red + 8);   // 8 ints
  const int g = blockIdx.x % b2, r = blockIdx.x / b2;
  const int tid = threadIdx.x;

  // the slice, A[p][s] = M[p*b2 + g][r*q1i + s]
  constexpr int VEC = 16 / sizeof(T);
  const T* src = M + static_cast<int64_t>(g) * in + static_cast<int64_t>(r) * q1i;
  if (q1i % VEC == 0 && in % VEC == 0) {
    const int per_row = q1i / VEC;
    for (int e = tid; e < q2o * per_row; e += PT) {
      const int p = e / per_row, s0 = (e % per_row) * VEC;
      const u32x4 raw = *reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(p) * b2 * in + s0);
      const T* el = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int j = 0; j < VEC; ++j) A[p * pitch + s0 + j] = Io<T>::load(el, j);
    }
  } else {
    for (int e = tid; e < q2o * q1i; e += PT) {
      const int p = e / q1i, s = e % q1i;
      A[p * pitch + s] = Io<T>::load(src, static_cast<int64_t>(p) * b2 * in + s);
    }
  }
  __syncthreads();

  const int tpr_rows = lanes_per_row(q2o), tpr_cols = lanes_per_row(q1i);
  // start: column sums of A (the unit vector e_0 if they vanish)
  for (int s = tid; s < q1i; s += PT) {
    float acc = 0.f;
    for (int p = 0; p < q2o; ++p) acc += A[p * pitch + s];
    v[s] = acc;
  }
  __syncthreads();
  float part = 0.f;
  for (int s = tid; s < q1i; s += PT) part += v[s] * v[s];
  float nrm = block_sum(part, red);
  if (!(nrm > 0.f)) {
    for (int s = tid; s < q1i; s += PT) v[s] = s == 0 ? 1.f : 0.f;
    nrm = 1.f;
  }
  float inv = 1.f / sqrtf(nrm);
  for (int s = tid; s < q1i; s += PT) v[s] *= inv;
  __syncthreads();

  for (int it = 0; it < iters; ++it) {
    matvec(A, pitch, 1, q2o, q1i, v, u, tpr_rows);   // u = A v
    __syncthreads();
    matvec(A, 1, pitch, q1i, q2o, u, v, tpr_cols);   // v = Aᵀ u
    __syncthreads();
    part = 0.f;
    for (int s = tid; s < q1i; s += PT) part += v[s] * v[s];
    nrm = block_sum(part, red);
    inv = nrm > 0.f ? 1.f / sqrtf(nrm) : 0.f;
    for (int s = tid; s < q1i; s += PT) v[s] *= inv;
    __syncthreads();
  }

  // u = A v, sigma = |u|
  matvec(A, pitch, 1, q2o, q1i, v, u, tpr_rows);
  __syncthreads();
  part = 0.f;
  for (int p = tid; p < q2o; p += PT) part += u[p] * u[p];
  const float sigma = sqrtf(block_sum(part, red));

  // sign: R's entry of largest magnitude (first on ties) is positive
  float best = -1.f;
  int besti = 0x7fffffff;
  for (int s = tid; s < q1i; s += PT) {
    const float a = fabsf(v[s]);
    if (a > best) best = a, besti = s;     // s increases: the first maximum wins
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ob = __shfl_xor(best, o);
    const int oi = __shfl_xor(besti, o);
    if (ob > best || (ob == best && oi < besti)) best = ob, besti = oi;
  }
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = best, ired[tid >> 6] = besti;
  __syncthreads();
  best = red[0];
  besti = ired[0];
  for (int w = 1; w < PT / 64; ++w)
    if (red[w] > best || (red[w] == best && ired[w] < besti)) best = red[w], besti = ired[w];
  const float sgn = v[besti] < 0.f ? -1.f : 1.f;

  const float rs = sqrtf(sigma);
  const float lscale = sigma > 0.f ? sgn / rs : 0.f;
  T* R = W1 + (static_cast<int64_t>(r) * b2 + g) * q1i;
  for (int s = tid; s < q1i; s += PT) Io<T>::store(R, s, sgn * rs * v[s]);
  T* L = W2 + static_cast<int64_t>(g) * q2o * b1 + r;
  for (int p = tid; p < q2o; p += PT) Io<T>::store(L, static_cast<int64_t>(p) * b1, lscale * u[p]);
}

// Square Q x Q slices (Q = 32, 64 or 128): the slice stays in registers. The
// 256 threads form a 16 x 16 grid; thread (tr, tc) holds the E x E sub-block
// (E = Q/16) at rows tr*E.., columns tc*E... A row strip is 16 adjacent
// lanes, a column strip is 16 lanes 16 apart (4 in each wave).
//  * u = A v: products against v's E entries, summed over the row strip
//    with shuffles; every thread of the strip then holds its E entries of u,
//    which is all the next product needs.
//  * v = Aᵀ u: products against u's E entries, summed over the wave's 4 row
//    strips with shuffles and over the 4 waves through LDS (double-buffered,
//    so one barrier per iteration); every thread then holds its E entries of
//    v, and |v|² is a shuffle sum over the 16 column strips of its wave.
// Same start, iteration count, normalisation and sign rule as the general
// kernel. bf16 slices of 64 or 128 instead form B = AᵀA once with MFMAs
// (the slice written transposed to LDS; exact products, fp32 sums) and take
// each power step as one product with B: w = B v by row strips, v = B w by
// column strips (B is symmetric), so an exchange round through LDS covers
// two steps; the final A v reads the bf16 copy in LDS.
template <typename T, int Qs>
__global__ __launch_bounds__(PT) void project_square_kernel(const T* __restrict__ M,
                                                            T* __restrict__ W1,
                                                            T* __restrict__ W2, int64_t in,
                                                            int b1, int b2, int iters) {
  constexpr int E = Qs / 16;
  __shared__ float part[2][4][Qs];   // per-wave column partials, double-buffered
  __shared__ float red[4];
  const int g = blockIdx.x % b2, r = blockIdx.x / b2;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int tr = tid >> 4, tc = tid & 15;
  float a[E][E];
  const T* src = M + static_cast<int64_t>(g) * in + static_cast<int64_t>(r) * Qs + tc * E;
  constexpr int VEC = 16 / sizeof(T);                 // elements per 16-byte load
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const T* rowp = src + static_cast<int64_t>(tr * E + i) * b2 * in;
    if constexpr (E % VEC == 0) {
#pragma unroll
      for (int j0 = 0; j0 < E; j0 += VEC) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(rowp + j0);
        const T* el = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int j = 0; j < VEC; ++j) a[i][j0 + j] = Io<T>::load(el, j);
      }
    } else {
#pragma unroll
      for (int j = 0; j < E; ++j) a[i][j] = Io<T>::load(rowp, j);
    }
  }

  // v[tc*E + j] = sum_p x[p] A[p][tc*E + j], x given by this thread's rows
  int buf = 0;
  auto colprod = [&](const float (&x)[E], float (&v)[E]) {
#pragma unroll
    for (int j = 0; j < E; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < E; ++i) acc += a[i][j] * x[i];
      acc += __shfl_xor(acc, 16);
      acc += __shfl_xor(acc, 32);
      v[j] = acc;
    }
    if (lane < 16) {
#pragma unroll
      for (int j = 0; j < E; ++j) part[buf][wv][tc * E + j] = v[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < E; ++j)
      v[j] = part[buf][0][tc * E + j] + part[buf][1][tc * E + j] + part[buf][2][tc * E + j] +
             part[buf][3][tc * E + j];
    buf ^= 1;
  };
  // |v|² over all Q entries (the 16 column strips of this wave)
  auto norm2 = [&](const float (&v)[E]) {
    float p2 = 0.f;
#pragma unroll
    for (int j = 0; j < E; ++j) p2 += v[j] * v[j];
    return row16_sum(p2);
  };
  // u = A v for this thread's rows
  auto rowprod = [&](const float (&v)[E], float (&u)[E]) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < E; ++j) acc += a[i][j] * v[j];
      u[i] = row16_sum(acc);
    }
  };

  float v[E], u[E];
  {
    float ones[E];
#pragma unroll
    for (int i = 0; i < E; ++i) ones[i] = 1.f;
    colprod(ones, v);                          // start: column sums
    const float nrm = norm2(v);
    if (nrm > 0.f) {
      const float inv = 1.f / sqrtf(nrm);
#pragma unroll
      for (int j = 0; j < E; ++j) v[j] *= inv;
    } else {
#pragma unroll
      for (int j = 0; j < E; ++j) v[j] = (tc * E + j == 0) ? 1.f : 0.f;
    }
  }
  if constexpr (std::is_same<T, uint16_t>::value && Qs >= 64) {
    // bf16: B = AᵀA once on MFMA (exact products, fp32 sums), then power
    // steps v <- B v, two per exchange round. Wave w keeps rows
    // [32w, 32w + 32) (Q = 128; [16w, 16w + 16) for 64) of B in the MFMA
    // result layout: lane holds B[16mt + 4lh + e][16nt + l15]. v lives by
    // columns (lane: v[16nt + l15]); w = B v by rows (lane: w[16mt + 4lh + e],
    // a 16-lane row sum); v = B w (B symmetric) sums over the wave's rows
    // with shuffles and over the waves through LDS.
    constexpr int AP = Qs + 8;           // LDS pitch of Aᵀ (bf16)
    constexpr int NT = Qs / 16, MTW = NT / 4;
    __shared__ __attribute__((aligned(16))) uint16_t ast[Qs * AP];   // Aᵀ[col][row]
    __shared__ float vs[Qs];
    const int l15 = lane & 15, lh = lane >> 4;
    // Aᵀ: column tc*E + j, rows tr*E .. tr*E + E - 1 (the bf16 values exactly)
#pragma unroll
    for (int j = 0; j < E; ++j) {
      uint32_t pk[E / 2];
#pragma unroll
      for (int i = 0; i < E / 2; ++i)
        pk[i] = (__float_as_uint(a[2 * i][j]) >> 16) | (__float_as_uint(a[2 * i + 1][j]) & 0xffff0000u);
      uint16_t* dst = &ast[(tc * E + j) * AP + tr * E];
      if constexpr (E == 8)
        *reinterpret_cast<u32x4*>(dst) = u32x4{pk[0], pk[1], pk[2], pk[3]};
      else
        *reinterpret_cast<u32x2*>(dst) = u32x2{pk[0], pk[1]};
    }
    if (tr == 0) {
#pragma unroll
      for (int j = 0; j < E; ++j) vs[tc * E + j] = v[j];
    }
    __syncthreads();
    f32x4 bacc[MTW][NT];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) bacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < Qs / 32; ++ks) {
      bf16x8 fa[MTW], fb[NT];
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt)
        fa[mt] = as_bf16x8(*reinterpret_cast<const u16x8*>(
            &ast[(16 * (MTW * wv + mt) + l15) * AP + 32 * ks + 8 * lh]));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        fb[nt] = as_bf16x8(*reinterpret_cast<const u16x8*>(&ast[(16 * nt + l15) * AP + 32 * ks + 8 * lh]));
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          bacc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[mt], fb[nt], bacc[mt][nt], 0, 0, 0);
    }
    float vc[NT], wr[MTW][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) vc[nt] = vs[16 * nt + l15];
    auto rowprod_b = [&]() {   // wr = B vc, rows of this wave
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float acc = 0.f;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc += bacc[mt][nt][e] * vc[nt];
          wr[mt][e] = row16_sum(acc);
        }
    };
    auto colprod_b = [&]() {   // vc = B wr (B symmetric), then normalised
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float acc = 0.f;
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc += bacc[mt][nt][e] * wr[mt][e];
        acc += __shfl_xor(acc, 16);
        acc += __shfl_xor(acc, 32);
        vc[nt] = acc;
      }
      if (lane < 16) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) part[buf][wv][16 * nt + l15] = vc[nt];
      }
      __syncthreads();
      float p2 = 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int c = 16 * nt + l15;
        vc[nt] = part[buf][0][c] + part[buf][1][c] + part[buf][2][c] + part[buf][3][c];
        p2 += vc[nt] * vc[nt];
      }
      buf ^= 1;
      const float nrm = row16_sum(p2);
      const float inv = nrm > 0.f ? 1.f / sqrtf(nrm) : 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) vc[nt] *= inv;
    };
    int left = iters;
    for (; left >= 2; left -= 2) {
      rowprod_b();   // w = B v (not normalised: one step's growth)
      colprod_b();   // v = B w, normalised
    }
    if (left == 1) {
      // one step: v by rows from the lanes that hold it by columns
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) wr[mt][e] = __shfl(vc[MTW * wv + mt], (lane & 48) | (4 * lh + e));
      colprod_b();
    }
    __syncthreads();   // every lane has read vs
    if (wv == 0 && lane < 16) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) vs[16 * nt + l15] = vc[nt];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < E; ++j) v[j] = vs[tc * E + j];
    // u = A v from the bf16 copy (A's registers are free after the start):
    // A[tr*E + i][tc*E + j] = Aᵀ[tc*E + j][tr*E + i]
    float pu[E];
#pragma unroll
    for (int i = 0; i < E; ++i) pu[i] = 0.f;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const uint16_t* col = &ast[(tc * E + j) * AP + tr * E];
      uint32_t w32[E / 2];
      if constexpr (E == 8) {
        const u32x4 q = *reinterpret_cast<const u32x4*>(col);
        w32[0] = q[0], w32[1] = q[1], w32[2] = q[2], w32[3] = q[3];
      } else {
        const u32x2 q = *reinterpret_cast<const u32x2*>(col);
        w32[0] = q[0], w32[1] = q[1];
      }
#pragma unroll
      for (int i = 0; i < E / 2; ++i) {
        pu[2 * i] += __uint_as_float(w32[i] << 16) * v[j];
        pu[2 * i + 1] += __uint_as_float(w32[i] & 0xffff0000u) * v[j];
      }
    }
#pragma unroll
    for (int i = 0; i < E; ++i) u[i] = row16_sum(pu[i]);
  } else {
    for (int it = 0; it < iters; ++it) {
      rowprod(v, u);                             // u = A v
      colprod(u, v);                             // v = Aᵀ u
      const float nrm = norm2(v);
      const float inv = nrm > 0.f ? 1.f / sqrtf(nrm) : 0.f;
#pragma unroll
      for (int j = 0; j < E; ++j) v[j] *= inv;
    }
    rowprod(v, u);
  }
  // sigma = |u|: this wave's 4 row strips, then the 4 waves
  float p2 = 0.f;
#pragma unroll
  for (int i = 0; i < E; ++i) p2 += u[i] * u[i];
  p2 += __shfl_xor(p2, 16);
  p2 += __shfl_xor(p2, 32);
  if (lane == 0) red[wv] = p2;
  __syncthreads();
  const float sigma = sqrtf(red[0] + red[1] + red[2] + red[3]);

  // sign: the entry of v of largest magnitude (first on ties) is positive
  float best = -1.f;
  int besti = 0x7fffffff;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const float av = fabsf(v[j]);
    if (av > best) best = av, besti = tc * E + j;
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    const float ob = __shfl_xor(best, o);
    const int oi = __shfl_xor(besti, o);
    if (ob > best || (ob == best && oi < besti)) best = ob, besti = oi;
  }
  float vb = 0.f;
#pragma unroll
  for (int j = 0; j < E; ++j) vb = (tc * E + j == besti) ? v[j] : vb;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    const float ov = __shfl_xor(vb, o);
    vb = (ov != 0.f) ? ov : vb;   // only the owner's lane holds it (v has besti's value there)
  }
  const float sgn = vb < 0.f ? -1.f : 1.f;
  const float rs = sqrtf(sigma);
  const float lscale = sigma > 0.f ? sgn / rs : 0.f;
  if (tr == 0) {
    T* R = W1 + (static_cast<int64_t>(r) * b2 + g) * Qs + tc * E;
#pragma unroll
    for (int j = 0; j < E; ++j) Io<T>::store(R, j, sgn * rs * v[j]);
  }
  if (tc == 0) {
    T* L = W2 + static_cast<int64_t>(g) * Qs * b1 + r;
#pragma unroll
    for (int i = 0; i < E; ++i) Io<T>::store(L, static_cast<int64_t>(tr * E + i) * b1, lscale * u[i]);
  }
}

}  // namespace

size_t project_lds_bytes(int64_t q1i, int64_t q2o) {
  return static_cast<size_t>(q2o * (q1i + 1) + q1i + q2o + 16) * sizeof(float);
}

hipError_t launch_project(const void* m, void* w1, void* w2, int64_t in, int64_t nb1,
                          int64_t nb2, int64_t q1i, int64_t q2o, int iters, bool bf16,
                          hipStream_t s) {
  const size_t lds = project_lds_bytes(q1i, q2o);
  const dim3 grid(static_cast<unsigned>(nb1 * nb2)), block(PT);
  if (q1i == q2o && (q1i == 32 || q1i == 64 || q1i == 128)) {
    const int b1 = static_cast<int>(nb1), b2 = static_cast<int>(nb2);
#define MONARCH_SQ_PROJECT(TT, QQ)                                                          \
  hipLaunchKernelGGL((project_square_kernel<TT, QQ>), grid, block, 0, s,                     \
                     static_cast<const TT*>(m), static_cast<TT*>(w1), static_cast<TT*>(w2), \
                     in, b1, b2, iters)
    if (bf16) {
      if (q1i == 32) MONARCH_SQ_PROJECT(uint16_t, 32);
      else if (q1i == 64) MONARCH_SQ_PROJECT(uint16_t, 64);
      else MONARCH_SQ_PROJECT(uint16_t, 128);
    } else {
      if (q1i == 32) MONARCH_SQ_PROJECT(float, 32);
      else if (q1i == 64) MONARCH_SQ_PROJECT(float, 64);
      else MONARCH_SQ_PROJECT(float, 128);
    }
#undef MONARCH_SQ_PROJECT
    return hipGetLastError();
  }
  if (bf16) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(project_slices_kernel<uint16_t>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(project_slices_kernel<uint16_t>, grid, block, lds, s,
                       static_cast<const uint16_t*>(m), static_cast<uint16_t*>(w1),
                       static_cast<uint16_t*>(w2), in, static_cast<int>(nb1),
                       static_cast<int>(nb2), static_cast<int>(q1i), static_cast<int>(q2o), iters);
  } else {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(project_slices_kernel<float>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(project_slices_kernel<float>, grid, block, lds, s,
                       static_cast<const float*>(m), static_cast<float*>(w1),
                       static_cast<float*>(w2), in, static_cast<int>(nb1), static_cast<int>(nb2),
                       static_cast<int>(q1i), static_cast<int>(q2o), iters);
  }
  return hipGetLastError();
}

}  // namespace monarch
