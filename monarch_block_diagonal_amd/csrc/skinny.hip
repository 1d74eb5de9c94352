// Block products with few rows and a long reduction (at most 16 rows, K of
// 128 or more), in fp32 or bf16:
//   C[i, col(j)] = act(sum_k A[i, k] B[row(j), k] + bias),   i < M <= 16,
// with both operands contiguous along k. At a batch of 10 the recommender
// MLP's first Monarch layer (10000 -> 1024 with 4 blocks; the "efficiency
// testing numbers" thread of the scatterbrain issues page) has a stage-1
// forward of this form: 10 rows, K = 2500, 256 outputs per block. Tiles
// sized for many rows leave such a product with 16 workgroups that each walk
// the whole K, so the launch is one long chain of dependent steps.
//
// Here a workgroup owns one block and 16 output columns, and its eight waves
// split K: wave w takes chunks [w*n/8, (w+1)*n/8) of the n chunks (16 k in
// fp32, 32 in bf16), each lane loading one 16-byte piece of its A row and
// one of its B row per chunk, eight chunks in flight. A chunk feeds four
// v_mfma_f32_16x16x4f32 (lane group lh supplies k = 4lh + e in the e-th) or
// one v_mfma_f32_16x16x32_bf16, accumulating in fp32. The eight partial
// 16 x 16 tiles are summed through LDS in wave order, so the result does not
// depend on timing; bias, ReLU and the I/O rounding follow. Rows past M read
// the last row and are not stored. Pieces may start at any 4-byte boundary
// (16-byte global loads need only dword alignment), so fp32 operands take
// any offsets and bf16 ones even element offsets.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace monarch {
namespace {

constexpr int kSkWaves = 8;
constexpr int kSkUnroll = 8;

typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
__device__ __forceinline__ u32x4 sk_ld16(const void* p) {
  const u32x4a4 v = *static_cast<const u32x4a4*>(p);
  return u32x4{v[0], v[1], v[2], v[3]};
}

template <typename T>
__device__ __forceinline__ float sk_to_f32(T v) {
  if constexpr (std::is_same<T, float>::value) return v;
  else return bf16_to_f32(v);
}

template <typename T>
__device__ __forceinline__ f32x4 sk_mfma(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (std::is_same<T, float>::value) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]), c,
                                               0, 0, 0);
    return c;
  } else {
    bf16x8 x, y;
    __builtin_memcpy(&x, &a, sizeof(x));
    __builtin_memcpy(&y, &b, sizeof(y));
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c, 0, 0, 0);
  }
}

template <typename T>
__global__ __launch_bounds__(kSkWaves * 64) void skinny_kernel(GemmArgs p) {
  constexpr int VEC = 16 / static_cast<int>(sizeof(T));   // elements per 16-byte piece
  constexpr int KC = 4 * VEC;                              // k per chunk
  __shared__ float part[kSkWaves][16][17];
  const int64_t blk = blockIdx.x % p.nblk;
  const int64_t j0 = static_cast<int64_t>(blockIdx.x / p.nblk) * 16;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l15 = lane & 15, lh = lane >> 4;

  // this block's K (zero padding cuts it short), in chunks
  int64_t K = p.K;
  if (p.k_lim >= 0) {
    const int64_t kv = p.k_lim - blk * p.k_lim_bs;
    K = K < kv ? K : kv;
  }
  if (K < 0) K = 0;
  const int64_t nfull = K / KC, nch = (K + KC - 1) / KC;
  const int64_t c0 = w * nch / kSkWaves, c1 = (w + 1) * nch / kSkWaves;
  const int64_t c1f = c1 < nfull ? c1 : nfull;   // chunks with every k in range

  const int64_t ai = l15 < p.M ? l15 : p.M - 1;
  const int64_t bj = j0 + l15 < p.N ? j0 + l15 : p.N - 1;
  const T* ap = static_cast<const T*>(p.A) + blk * p.a_sb + ai * p.a_si + lh * VEC;
  const T* bp = static_cast<const T*>(p.B) + blk * p.b_sb +
                col_off(bj, p.nsplit, p.b_sj_hi, p.b_sj) + lh * VEC;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int64_t c = c0;
  for (; c + kSkUnroll <= c1f; c += kSkUnroll) {
    u32x4 va[kSkUnroll], vb[kSkUnroll];
#pragma unroll
    for (int u = 0; u < kSkUnroll; ++u) {
      va[u] = sk_ld16(ap + (c + u) * KC);
      vb[u] = sk_ld16(bp + (c + u) * KC);
    }
#pragma unroll
    for (int u = 0; u < kSkUnroll; ++u) acc = sk_mfma<T>(va[u], vb[u], acc);
  }
  for (; c < c1f; ++c) acc = sk_mfma<T>(sk_ld16(ap + c * KC), sk_ld16(bp + c * KC), acc);
  if (c < c1) {
    // the last, partial chunk: element loads, zeros past K
    T ea[VEC], eb[VEC];
    const int64_t kb = c * KC + lh * VEC;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const bool in = kb + e < K;
      ea[e] = in ? ap[c * KC + e] : T(0);
      eb[e] = in ? bp[c * KC + e] : T(0);
    }
    u32x4 va, vb;
    __builtin_memcpy(&va, ea, 16);
    __builtin_memcpy(&vb, eb, 16);
    acc = sk_mfma<T>(va, vb, acc);
  }

  // lane holds the partial C[4lh + v][l15]; sum the waves' tiles in order
#pragma unroll
  for (int v = 0; v < 4; ++v) part[w][4 * lh + v][l15] = acc[v];
  __syncthreads();
  if (tid < 256) {
    const int i = tid >> 4, jl = tid & 15;
    const int64_t j = j0 + jl;
    if (i < p.M && j < p.N) {
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < kSkWaves; ++q) s += part[q][i][jl];
      const int64_t off = blk * p.c_sb + col_off(j, p.nsplit, p.c_sj_hi, p.c_sj);
      if (p.c_cols < 0 || off < p.c_cols) {
        if (p.bias) s += sk_to_f32(static_cast<const T*>(p.bias)[off]);
        if (p.relu) s = s > 0.f ? s : 0.f;
        T* C = static_cast<T*>(p.C) + i * p.c_si + off;
        if constexpr (std::is_same<T, float>::value) *C = s;
        else *C = f32_to_bf16(s);
      }
    }
  }
}

bool even(int64_t v) { return (v & 1) == 0; }

}  // namespace

bool skinny_ok(const GemmArgs& a, bool bf16) {
  if (a.partial || a.accum || a.mask || a.n_lim >= 0) return false;
  if (a.M < 1 || a.M > 16 || a.K < 128 || a.N < 1 || a.nblk < 1) return false;
  if (a.a_sk != 1 || a.b_sk != 1) return false;
  if (bf16) {
    // 16-byte pieces at 4-byte alignment: even element offsets
    const auto p4 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 3) == 0; };
    if (!p4(a.A) || !p4(a.B)) return false;
    if (!even(a.a_si) || !even(a.a_sb) || !even(a.b_sb) || !even(a.b_sj)) return false;
    if (a.nsplit > 0 && !even(a.b_sj_hi)) return false;
  }
  return true;
}

hipError_t launch_skinny(const GemmArgs& a, bool bf16, hipStream_t s) {
  const int64_t grid = a.nblk * ((a.N + 15) / 16);
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 g(static_cast<unsigned>(grid)), b(kSkWaves * 64);
  if (bf16)
    hipLaunchKernelGGL(skinny_kernel<uint16_t>, g, b, 0, s, a);
  else
    hipLaunchKernelGGL(skinny_kernel<float>, g, b, 0, s, a);
  return hipGetLastError();
}

}  // namespace monarch
