// Dense -> Monarch projection (Definition C.3 case, out = nblocks1 * nblocks2).
//
// The scatterbrain issues page ("projection" thread) rearranges M as
// '(p k) (r s) -> k r p s' and fits every (k, r) slice on its own; the
// Monarch paper's abstract calls the result an analytical optimal solution.
// With w1 = R [b1, b2, q1i] and w2 = L [b2, q2o, b1], slice (g, r) over (p, s)
// is A[p][s] = M[p*b2 + g][r*q1i + s] and the Monarch matrix holds
// L[g, p, r] * R[r, g, s] there, so the nearest Monarch matrix takes each
// slice's nearest rank-one matrix sigma * u * vᵀ (top singular triple,
// Eckart-Young). For a unit vector x the rank-one fit (A x) xᵀ leaves the
// error ||A||² - xᵀ B x with B = AᵀA, so the fit is optimal exactly when x
// maximises the Rayleigh quotient of B.
//
// Method: Lanczos on B = AᵀA (B never formed: each step is u = A v, w = Aᵀ u)
// with full reorthogonalisation (classical Gram-Schmidt, twice) against the
// cycle's basis, in fp32. A cycle of up to KC steps (fewer on breakdown, when
// the Krylov space is exhausted) gives the tridiagonal T = VᵀBV; its top
// eigenvalue is bracketed by multisection on Sturm counts (64 lanes, fp32),
// and its eigenvector s by two steps of inverse iteration with the shift just
// above that bracket, where shift·I - T is positive definite, so the
// tridiagonal solve needs no pivoting (fp64). The Ritz vector x = V s is
// accepted when ||B x - theta x|| <= kProjectTol * theta (theta = xᵀBx),
// else the next cycle restarts from x, until the caller's step budget is
// spent; each slice reports the products it used, or 0 if it did not converge. Lanczos reaches the top
// pair at a rate set by the square root of the spectral gap, and a cluster
// of near-equal top values is harmless: any unit vector in its span is a fit
// within the cluster's width of the optimum.
//
// One workgroup per slice, the slice zero-padded to QP x QP (QP = 16, 32, 64
// or 128; padding changes no singular triple) and held in registers: the 256
// threads form a 16 x 16 grid, thread (tr, tc) holding the E x E sub-block
// (E = QP/16) at rows tr*E.., columns tc*E... Vectors indexed by columns are
// held by column strips (thread (tr, tc) keeps entries tc*E..), replicated
// over tr; a row strip is 16 adjacent lanes (sums over it are DPP row sums),
// sums over the 16 row strips take shuffles within a wave and one exchange
// through LDS between the 4 waves. The Lanczos basis lives in LDS; in the
// Gram-Schmidt passes row strip tr handles the basis vectors j = tr (mod 16).
// The result is split evenly, L[g, :, r] = A x / sqrt(sigma),
// R[r, g, :] = sqrt(sigma) x, with the sign chosen so that R's entry of
// largest magnitude (the first one on ties) is positive.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace monarch {
namespace {

constexpr int PT = 256;                 // threads per workgroup (16 x 16 grid)
constexpr int KC = 32;                  // Lanczos steps per cycle at most
constexpr float kProjectTol = 1e-4f;    // accept x when ||B x - theta x|| <= tol * theta
constexpr float kBreakdown = 1e-6f;     // end a cycle when beta <= this * max |alpha|

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

// Number of eigenvalues below x of the symmetric tridiagonal matrix with
// diagonal al[0..m) and off-diagonal be[0..m-1): the negative pivots of the
// LDLᵀ factorisation of T - x I (Sturm sequence), in fp32.
__device__ int sturm_count(const float* al, const float* be, int m, float x) {
  int cnt = 0;
  float d = 1.f;
  for (int i = 0; i < m; ++i) {
    d = (al[i] - x) - (i ? be[i - 1] * be[i - 1] * __builtin_amdgcn_rcpf(d) : 0.f);
    if (d == 0.f) d = -1e-30f;
    cnt += d < 0.f ? 1 : 0;
  }
  return cnt;
}

// Top eigenvector of the m x m tridiagonal T (al, be in LDS) into s[0..m),
// by wave 0 (all 64 lanes call it). The top eigenvalue is bracketed by
// multisection: each round the 64 lanes take Sturm counts at 64 points of
// (lo, hi), keeping count(lo) < m = count(hi). Lane 0 then runs two steps of
// inverse iteration with the shift just above hi, where shift·I - T is
// positive definite (LDLᵀ without pivoting, fp64; tw: 2*KC doubles of LDS).
__device__ void tridiag_top(const float* al, const float* be, int m, float* s, double* tw,
                            int lane) {
  if (m == 1) {
    if (lane == 0) s[0] = 1.f;
    return;
  }
  float lo = al[0], hi = -3.0e38f;
  for (int i = 0; i < m; ++i) {
    lo = fmaxf(lo, al[i]);
    const float rad = (i ? fabsf(be[i - 1]) : 0.f) + (i + 1 < m ? fabsf(be[i]) : 0.f);
    hi = fmaxf(hi, al[i] + rad);
  }
  hi += fmaxf(fabsf(hi) * 1e-6f, 1e-30f);          // strictly above every eigenvalue
  for (int round = 0; round < 12; ++round) {
    const float x = lo + (hi - lo) * static_cast<float>(lane + 1) * (1.f / 65.f);
    const bool above = sturm_count(al, be, m, x) >= m;
    const uint64_t mask = __ballot(above);
    float nlo, nhi;
    if (mask) {
      const int l = __builtin_ctzll(mask);
      nhi = __shfl(x, l);
      nlo = l > 0 ? __shfl(x, l - 1) : lo;
    } else {
      nlo = __shfl(x, 63);
      nhi = hi;
    }
    lo = nlo, hi = nhi;
    if (hi - lo <= fabsf(hi) * 2.4e-7f) break;
  }
  if (lane == 0) {
    const double sh = static_cast<double>(hi) + fmax(fabs(static_cast<double>(hi)) * 1e-6, 1e-30);
    double* c = tw;          // elimination multipliers
    double* y = tw + KC;     // right-hand side, then solution
    for (int i = 0; i < m; ++i) y[i] = 1.0;
    for (int it = 0; it < 2; ++it) {
      // (sh I - T) y = rhs: diagonal sh - al[i] > 0, off-diagonal -be[i]
      double den = sh - al[0];
      c[0] = -static_cast<double>(be[0]) / den;
      y[0] = y[0] / den;
      for (int i = 1; i < m; ++i) {
        const double e = -static_cast<double>(be[i - 1]);
        den = (sh - al[i]) - e * c[i - 1];
        c[i] = i + 1 < m ? -static_cast<double>(be[i]) / den : 0.0;
        y[i] = (y[i] - e * y[i - 1]) / den;
      }
      for (int i = m - 2; i >= 0; --i) y[i] -= c[i] * y[i + 1];
      double n2 = 0.0;
      for (int i = 0; i < m; ++i) n2 += y[i] * y[i];
      const double inv = n2 > 0.0 ? 1.0 / sqrt(n2) : 0.0;
      for (int i = 0; i < m; ++i) y[i] *= inv;
    }
    for (int i = 0; i < m; ++i) s[i] = static_cast<float>(y[i]);
  }
}

template <typename T, int QP>
__global__ __launch_bounds__(PT) void project_lanczos_kernel(
    const T* __restrict__ M, T* __restrict__ W1, T* __restrict__ W2, int* __restrict__ status,
    int64_t in, int b1, int b2, int q1i, int q2o, int max_steps) {
  constexpr int E = QP / 16;
  __shared__ float part[2][4][QP];        // per-wave column partial sums, double-buffered
  __shared__ float vb[KC + 1][QP];        // the cycle's Lanczos basis
  __shared__ float tal[KC], tbe[KC], ts[KC];
  __shared__ double tw[2 * KC];
  const int g = blockIdx.x % b2, r = blockIdx.x / b2;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int tr = tid >> 4, tc = tid & 15;

  // the slice A[p][s] = M[p*b2 + g][r*q1i + s], zero-padded to QP x QP
  float a[E][E];
  const T* src = M + static_cast<int64_t>(g) * in + static_cast<int64_t>(r) * q1i;
  constexpr int VEC = 16 / sizeof(T);
  const bool vec = q1i == QP && q2o == QP && E % VEC == 0 && in % VEC == 0;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int p = tr * E + i;
    const T* rowp = src + static_cast<int64_t>(p) * b2 * in + tc * E;
    if (vec) {
#pragma unroll
      for (int j0 = 0; j0 < E; j0 += VEC) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(rowp + j0);
        const T* el = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int j = 0; j < VEC; ++j) a[i][j0 + j] = Io<T>::load(el, j);
      }
    } else {
#pragma unroll
      for (int j = 0; j < E; ++j)
        a[i][j] = (p < q2o && tc * E + j < q1i) ? Io<T>::load(rowp, j) : 0.f;
    }
  }

  int buf = 0;
  // x: this thread's partial over its rows -> the sums over all rows, per column
  auto colsum = [&](float(&x)[E]) {
#pragma unroll
    for (int j = 0; j < E; ++j) {
      x[j] += __shfl_xor(x[j], 16);
      x[j] += __shfl_xor(x[j], 32);
    }
    if (lane < 16) {
#pragma unroll
      for (int j = 0; j < E; ++j) part[buf][wv][tc * E + j] = x[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int c = tc * E + j;
      x[j] = part[buf][0][c] + part[buf][1][c] + part[buf][2][c] + part[buf][3][c];
    }
    buf ^= 1;
  };
  auto dot = [&](const float(&x)[E], const float(&y)[E]) {
    float p = 0.f;
#pragma unroll
    for (int j = 0; j < E; ++j) p += x[j] * y[j];
    return row16_sum(p);
  };
  auto rowprod = [&](const float(&v)[E], float(&u)[E]) {   // u = A v (this thread's rows)
#pragma unroll
    for (int i = 0; i < E; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < E; ++j) acc += a[i][j] * v[j];
      u[i] = row16_sum(acc);
    }
  };
  auto colprod = [&](const float(&u)[E], float(&w)[E]) {   // w = Aᵀ u
#pragma unroll
    for (int j = 0; j < E; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < E; ++i) acc += a[i][j] * u[i];
      w[j] = acc;
    }
    colsum(w);
  };
  auto normalize = [&](float(&x)[E]) {
    const float n2 = dot(x, x);
    const float inv = n2 > 0.f ? 1.f / sqrtf(n2) : 0.f;
#pragma unroll
    for (int j = 0; j < E; ++j) x[j] *= inv;
    return n2 > 0.f;
  };

  // ||A||² and the start vector: the column sums of |A| (nonzero when A is)
  float x[E];
  float fro2;
  {
    float f = 0.f;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        acc += fabsf(a[i][j]);
        f += a[i][j] * a[i][j];
      }
      x[j] = acc;
    }
    colsum(x);
    float fx[E];
#pragma unroll
    for (int j = 0; j < E; ++j) fx[j] = j ? 0.f : row16_sum(f);
    colsum(fx);
    fro2 = fx[0];
  }
  if (!normalize(x)) {
#pragma unroll
    for (int j = 0; j < E; ++j) x[j] = tc * E + j == 0 ? 1.f : 0.f;
  }

  int steps = 0, cycle = 0;
  bool conv = false;
  float theta = 0.f, u[E];
  for (;;) {
    // one Lanczos cycle from x
    const int kmax = min(KC, max(max_steps - steps, 1));
    float v[E];
#pragma unroll
    for (int j = 0; j < E; ++j) v[j] = x[j];
    if (tr == 0) {
#pragma unroll
      for (int j = 0; j < E; ++j) vb[0][tc * E + j] = v[j];
    }
    float amax = 0.f;
    int m = 0;
    for (int i = 0; i < kmax; ++i) {
      float uu[E], w[E];
      rowprod(v, uu);
      colprod(uu, w);
      const float al = dot(v, w);
      amax = fmaxf(amax, fabsf(al));
      // w -= V (Vᵀ w), twice; row strip tr takes basis vectors tr, tr + 16
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        float corr[E];
#pragma unroll
        for (int j = 0; j < E; ++j) corr[j] = 0.f;
        for (int jj = tr; jj <= i; jj += 16) {
          const float* vj = &vb[jj][tc * E];
          float p = 0.f;
#pragma unroll
          for (int j = 0; j < E; ++j) p += vj[j] * w[j];
          const float c = row16_sum(p);
#pragma unroll
          for (int j = 0; j < E; ++j) corr[j] += c * vj[j];
        }
        colsum(corr);
#pragma unroll
        for (int j = 0; j < E; ++j) w[j] -= corr[j];
      }
      const float be = sqrtf(dot(w, w));
      if (tid == 0) tal[i] = al, tbe[i] = be;
      m = i + 1;
      ++steps;
      if (i + 1 == kmax || !(be > kBreakdown * amax)) break;
      const float inv = 1.f / be;
#pragma unroll
      for (int j = 0; j < E; ++j) v[j] = w[j] * inv;
      if (tr == 0) {
#pragma unroll
        for (int j = 0; j < E; ++j) vb[i + 1][tc * E + j] = v[j];
      }
    }
    __syncthreads();   // T complete
    if (wv == 0) tridiag_top(tal, tbe, m, ts, tw, lane);
    __syncthreads();
    // Ritz vector x = V s
    {
      float xr[E];
#pragma unroll
      for (int j = 0; j < E; ++j) xr[j] = 0.f;
      for (int jj = tr; jj < m; jj += 16) {
        const float sj = ts[jj];
#pragma unroll
        for (int j = 0; j < E; ++j) xr[j] += sj * vb[jj][tc * E + j];
      }
      colsum(xr);
      if (normalize(xr)) {
#pragma unroll
        for (int j = 0; j < E; ++j) x[j] = xr[j];
      }
    }
    // accept x when B x is theta x to the tolerance
    float w[E], res[E];
    rowprod(x, u);
    colprod(u, w);
    theta = dot(x, w);
#pragma unroll
    for (int j = 0; j < E; ++j) res[j] = w[j] - theta * x[j];
    const float rho = sqrtf(dot(res, res));
    ++steps;
    ++cycle;
    conv = theta > 0.f ? rho <= kProjectTol * theta : fro2 == 0.f;
    if (conv || steps >= max_steps) break;
    if (!(theta > 0.f)) {
      // x fell in A's null space (only for contrived inputs): next unit vector
#pragma unroll
      for (int j = 0; j < E; ++j) x[j] = tc * E + j == cycle % q1i ? 1.f : 0.f;
    }
    __syncthreads();   // every thread is done with vb and ts before the next cycle
  }

  const float sigma = theta > 0.f ? sqrtf(theta) : 0.f;   // ||A x||
  // sign: the entry of x of largest magnitude (first on ties) is positive
  float best = -1.f;
  int besti = 0x7fffffff;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const float av = fabsf(x[j]);
    if (av > best) best = av, besti = tc * E + j;
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    const float ob = __shfl_xor(best, o);
    const int oi = __shfl_xor(besti, o);
    if (ob > best || (ob == best && oi < besti)) best = ob, besti = oi;
  }
  float vbest = 0.f;
#pragma unroll
  for (int j = 0; j < E; ++j) vbest = tc * E + j == besti ? x[j] : vbest;
  vbest = row16_sum(vbest);   // only the owning lane contributes
  const float sgn = vbest < 0.f ? -1.f : 1.f;
  const float rs = sqrtf(sigma);
  const float lscale = sigma > 0.f ? sgn / rs : 0.f;
  if (tr == 0) {
    T* R = W1 + (static_cast<int64_t>(r) * b2 + g) * q1i;
#pragma unroll
    for (int j = 0; j < E; ++j)
      if (tc * E + j < q1i) Io<T>::store(R, tc * E + j, sgn * rs * x[j]);
  }
  if (tc == 0) {
    T* L = W2 + static_cast<int64_t>(g) * q2o * b1 + r;
#pragma unroll
    for (int i = 0; i < E; ++i)
      if (tr * E + i < q2o) Io<T>::store(L, static_cast<int64_t>(tr * E + i) * b1, lscale * u[i]);
  }
  if (status && tid == 0) status[blockIdx.x] = conv ? steps : 0;
}

}  // namespace

int project_pad(int64_t q1i, int64_t q2o) {
  const int64_t q = q1i > q2o ? q1i : q2o;
  if (q <= 16) return 16;
  if (q <= 32) return 32;
  if (q <= 64) return 64;
  if (q <= 128) return 128;
  return 0;
}

hipError_t launch_project(const void* m, void* w1, void* w2, int* status, int64_t in,
                          int64_t nb1, int64_t nb2, int64_t q1i, int64_t q2o, int max_steps,
                          bool bf16, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(nb1 * nb2)), block(PT);
  const int b1 = static_cast<int>(nb1), b2 = static_cast<int>(nb2);
  const int qi = static_cast<int>(q1i), qo = static_cast<int>(q2o);
#define MONARCH_PROJECT(TT, QQ)                                                                 \
  hipLaunchKernelGGL((project_lanczos_kernel<TT, QQ>), grid, block, 0, s,                        \
                     static_cast<const TT*>(m), static_cast<TT*>(w1), static_cast<TT*>(w2),     \
                     status, in, b1, b2, qi, qo, max_steps)
  switch (project_pad(q1i, q2o) * (bf16 ? -1 : 1)) {
    case 16: MONARCH_PROJECT(float, 16); break;
    case 32: MONARCH_PROJECT(float, 32); break;
    case 64: MONARCH_PROJECT(float, 64); break;
    case 128: MONARCH_PROJECT(float, 128); break;
    case -16: MONARCH_PROJECT(uint16_t, 16); break;
    case -32: MONARCH_PROJECT(uint16_t, 32); break;
    case -64: MONARCH_PROJECT(uint16_t, 64); break;
    case -128: MONARCH_PROJECT(uint16_t, 128); break;
    default: return hipErrorInvalidValue;
  }
#undef MONARCH_PROJECT
  return hipGetLastError();
}

}  // namespace monarch
