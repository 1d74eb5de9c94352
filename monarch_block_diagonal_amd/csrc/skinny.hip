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
//
// The same scheme with 64 x 64 tiles (4 x 4 fragments per wave, the eight
// partial tiles summed through 130 KB of LDS) takes fp32 products with more
// rows but few tiles and a long K, e.g. the same layer at a batch of 1000
// (256 tiles, K = 2500): the tiled GEMM runs one four-wave workgroup per CU
// there, a wave per SIMD behind a barrier every K step, while here eight
// waves per CU stream their own K ranges with no barrier until the sum.
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

__device__ __forceinline__ f32x4 sk_mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  bf16x8 x, y;
  __builtin_memcpy(&x, &a, sizeof(x));
  __builtin_memcpy(&y, &b, sizeof(y));
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c, 0, 0, 0);
}

template <typename T, int FM, int FN>
__global__ __launch_bounds__(kSkWaves * 64) void skinny_kernel(GemmArgs p, int64_t n_tiles) {
  constexpr int VEC = 16 / static_cast<int>(sizeof(T));   // elements per 16-byte piece
  constexpr int KC = 4 * VEC;                              // k per chunk
  constexpr int TM = 16 * FM, TN = 16 * FN;
  constexpr int U = FM * FN == 1 ? kSkUnroll : 4;          // chunks in flight
  __shared__ float part[kSkWaves][TM][TN + 1];
  const int64_t blk = blockIdx.x % p.nblk;
  const int64_t t = blockIdx.x / p.nblk;
  const int64_t j0 = (t % n_tiles) * TN, i0 = (t / n_tiles) * TM;
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

  const T* ap[FM];
  const T* bp[FN];
#pragma unroll
  for (int mi = 0; mi < FM; ++mi) {
    const int64_t r = i0 + 16 * mi + l15;
    ap[mi] = static_cast<const T*>(p.A) + blk * p.a_sb + (r < p.M ? r : p.M - 1) * p.a_si + lh * VEC;
  }
#pragma unroll
  for (int ni = 0; ni < FN; ++ni) {
    const int64_t r = j0 + 16 * ni + l15;
    bp[ni] = static_cast<const T*>(p.B) + blk * p.b_sb +
             col_off(r < p.N ? r : p.N - 1, p.nsplit, p.b_sj_hi, p.b_sj) + lh * VEC;
  }

  f32x4 acc[FM][FN];
#pragma unroll
  for (int mi = 0; mi < FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
  // fp32: the e-th product of every fragment pair before the (e+1)-th, so
  // FM*FN independent accumulators separate two products into one of them
  auto mul = [&](const u32x4 (&va)[FM], const u32x4 (&vb)[FN]) {
    if constexpr (std::is_same<T, float>::value) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int mi = 0; mi < FM; ++mi)
#pragma unroll
          for (int ni = 0; ni < FN; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                __uint_as_float(va[mi][e]), __uint_as_float(vb[ni][e]), acc[mi][ni], 0, 0, 0);
    } else {
#pragma unroll
      for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < FN; ++ni) acc[mi][ni] = sk_mfma_bf16(va[mi], vb[ni], acc[mi][ni]);
    }
  };
  int64_t c = c0;
  for (; c + U <= c1f; c += U) {
    u32x4 va[U][FM], vb[U][FN];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int mi = 0; mi < FM; ++mi) va[u][mi] = sk_ld16(ap[mi] + (c + u) * KC);
#pragma unroll
      for (int ni = 0; ni < FN; ++ni) vb[u][ni] = sk_ld16(bp[ni] + (c + u) * KC);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) mul(va[u], vb[u]);
  }
  for (; c < c1f; ++c) {
    u32x4 va[FM], vb[FN];
#pragma unroll
    for (int mi = 0; mi < FM; ++mi) va[mi] = sk_ld16(ap[mi] + c * KC);
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) vb[ni] = sk_ld16(bp[ni] + c * KC);
    mul(va, vb);
  }
  if (c < c1) {
    // the last, partial chunk: element loads, zeros past K
    const int64_t kb = c * KC + lh * VEC;
    u32x4 va[FM], vb[FN];
#pragma unroll
    for (int mi = 0; mi < FM; ++mi) {
      T e[VEC];
#pragma unroll
      for (int q = 0; q < VEC; ++q) e[q] = kb + q < K ? ap[mi][c * KC + q] : T(0);
      __builtin_memcpy(&va[mi], e, 16);
    }
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) {
      T e[VEC];
#pragma unroll
      for (int q = 0; q < VEC; ++q) e[q] = kb + q < K ? bp[ni][c * KC + q] : T(0);
      __builtin_memcpy(&vb[ni], e, 16);
    }
    mul(va, vb);
  }

  // lane holds the partial C[16mi + 4lh + v][16ni + l15]; sum the waves'
  // tiles in order
#pragma unroll
  for (int mi = 0; mi < FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < FN; ++ni)
#pragma unroll
      for (int v = 0; v < 4; ++v) part[w][16 * mi + 4 * lh + v][16 * ni + l15] = acc[mi][ni][v];
  __syncthreads();
  for (int id = tid; id < TM * TN; id += kSkWaves * 64) {
    const int il = id / TN, jl = id - il * TN;
    const int64_t i = i0 + il, j = j0 + jl;
    if (i < p.M && j < p.N) {
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < kSkWaves; ++q) s += part[q][il][jl];
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

int skinny_mode(const GemmArgs& a, bool bf16) {
  if (a.partial || a.accum || a.mask || a.n_lim >= 0) return 0;
  if (a.M < 1 || a.N < 1 || a.nblk < 1 || a.K < 128) return 0;
  if (a.a_sk != 1 || a.b_sk != 1) return 0;
  if (bf16) {
    // 16-byte pieces at 4-byte alignment: even element offsets
    const auto p4 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 3) == 0; };
    if (!p4(a.A) || !p4(a.B)) return 0;
    if (!even(a.a_si) || !even(a.a_sb) || !even(a.b_sb) || !even(a.b_sj)) return 0;
    if (a.nsplit > 0 && !even(a.b_sj_hi)) return 0;
  }
  if (a.M <= 16) return 1;
  // fp32, K >= 512, at most 512 tiles of 64 x 64
  const int64_t tiles = ((a.M + 63) / 64) * ((a.N + 63) / 64) * a.nblk;
  if (!bf16 && a.K >= 512 && tiles <= 512) return 2;
  return 0;
}

hipError_t launch_skinny(const GemmArgs& a, int mode, bool bf16, hipStream_t s) {
  const int64_t tn = mode == 1 ? 16 : 64;
  const int64_t n_tiles = (a.N + tn - 1) / tn;
  const int64_t grid = a.nblk * n_tiles * ((a.M + tn - 1) / tn);
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 g(static_cast<unsigned>(grid)), b(kSkWaves * 64);
  if (mode == 1) {
    if (bf16)
      hipLaunchKernelGGL((skinny_kernel<uint16_t, 1, 1>), g, b, 0, s, a, n_tiles);
    else
      hipLaunchKernelGGL((skinny_kernel<float, 1, 1>), g, b, 0, s, a, n_tiles);
  } else if (mode == 2 && !bf16) {
    hipLaunchKernelGGL((skinny_kernel<float, 4, 4>), g, b, 0, s, a, n_tiles);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace monarch
