// Generic strided batched GEMM for any Monarch shape (gfx950).
//
// Each step of the two-stage Monarch product (Monarch paper, abstract: two
// block-diagonal factors; scatterbrain issues page, "hypercube" thread: each
// factor is a batch of independent matrix products, with the stride
// permutation between them) is a batch of independent block GEMMs whose
// operands sit at affine offsets. This kernel takes those offsets as strides,
// so the permutation costs nothing beyond the address arithmetic. It handles
// ragged tiles in every dimension and is the path for shapes without a
// specialised kernel (tiny blocks, odd block sizes such as 625 or 2500).
//
// Tile: 64x64 outputs per 256-thread workgroup, K step 32, operands staged in
// LDS; each of the 4 waves owns a 32x32 quarter computed with 16x16 MFMAs
// (fp32: v_mfma_f32_16x16x4_f32, full fp32 products and sums; bf16:
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace monarch {
namespace {

constexpr int BM = kGenBM, BN = kGenBN, BK = kGenBK;

template <typename T>
__global__ __launch_bounds__(256) void generic_gemm_kernel(GemmArgs p, int64_t m_tiles,
                                                           int64_t n_tiles, int a_k_fast,
                                                           int b_k_fast) {
  constexpr bool kBf16 = std::is_same<T, uint16_t>::value;
  constexpr int LD = kBf16 ? BK + 8 : BK + 1;  // row pitch in elements
  __shared__ __attribute__((aligned(16))) T As[BM * LD];
  __shared__ __attribute__((aligned(16))) T Bs[BN * LD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  int64_t t = blockIdx.x;
  const int64_t nt = t % n_tiles;
  t /= n_tiles;
  const int64_t mt = t % m_tiles;
  t /= m_tiles;
  const int64_t blk = t % p.nblk;
  const int64_t split = t / p.nblk;
  const int64_t kb = p.partial ? split * p.k_chunk : 0;
  const int64_t ke = p.partial ? (kb + p.k_chunk < p.K ? kb + p.k_chunk : p.K) : p.K;
  const int64_t i0 = mt * BM, j0 = nt * BN;

  const T* __restrict__ A = static_cast<const T*>(p.A);
  const T* __restrict__ B = static_cast<const T*>(p.B);

  f32x4 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = kb; k0 < ke; k0 += BK) {
    // A tile (i, k) -> As[i][k]; walk the dimension with the smaller stride fastest
    for (int e = tid; e < BM * BK; e += 256) {
      int i, k;
      if (a_k_fast) {
        k = e % BK;
        i = e / BK;
      } else {
        i = e % BM;
        k = e / BM;
      }
      const int64_t gi = i0 + i, gk = k0 + k;
      T v = T(0);
      if (gi < p.M && gk < ke) {
        const int64_t off = blk * p.a_sb + gi * p.a_si + gk * p.a_sk;
        v = A[off];
        if (p.mask && !(Io<T>::load(p.mask, off) > 0.f)) v = T(0);
      }
      As[i * LD + k] = v;
    }
    // B tile (k, j) -> Bs[j][k]
    for (int e = tid; e < BK * BN; e += 256) {
      int j, k;
      if (b_k_fast) {
        k = e % BK;
        j = e / BK;
      } else {
        j = e % BN;
        k = e / BN;
      }
      const int64_t gj = j0 + j, gk = k0 + k;
      T v = T(0);
      if (gj < p.N && gk < ke) v = B[blk * p.b_sb + gk * p.b_sk + col_off(gj, p.nsplit, p.b_sj_hi, p.b_sj)];
      Bs[j * LD + k] = v;
    }
    __syncthreads();

    if constexpr (kBf16) {
      // 16x16x32: lane supplies row (lane%16) and 8 consecutive k (group lane/16)
      bf16x8 a[2], b[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const u16x8 v = *reinterpret_cast<const u16x8*>(
            &As[(wm * 32 + mi * 16 + (lane & 15)) * LD + (lane >> 4) * 8]);
        a[mi] = as_bf16x8(v);
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const u16x8 v = *reinterpret_cast<const u16x8*>(
            &Bs[(wn * 32 + ni * 16 + (lane & 15)) * LD + (lane >> 4) * 8]);
        b[ni] = as_bf16x8(v);
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    } else {
#pragma unroll
      for (int ks = 0; ks < BK; ks += 4) {
        float a[2], b[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
          a[mi] = As[(wm * 32 + mi * 16 + (lane & 15)) * LD + ks + (lane >> 4)];
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          b[ni] = Bs[(wn * 32 + ni * 16 + (lane & 15)) * LD + ks + (lane >> 4)];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // 16x16 result layout: lane holds rows 4*(lane/16)+v, column lane%16
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t i = i0 + wm * 32 + mi * 16 + 4 * (lane >> 4) + v;
        const int64_t j = j0 + wn * 32 + ni * 16 + (lane & 15);
        if (i < p.M && j < p.N) {
          float val = acc[mi][ni][v];
          if (p.partial) {
            p.partial[((split * p.nblk + blk) * p.M + i) * p.N + j] = val;
          } else {
            if (p.relu) val = val > 0.f ? val : 0.f;
            Io<T>::store(p.C, blk * p.c_sb + i * p.c_si + col_off(j, p.nsplit, p.c_sj_hi, p.c_sj), val);
          }
        }
      }
}

// Elements [0, nA) of the flattened index space reduce partialA, the rest
// partialB.
template <typename T>
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float* __restrict__ wsA,
                                                              void* outA, int64_t nA,
                                                              int64_t splitsA,
                                                              const float* __restrict__ wsB,
                                                              void* outB, int64_t nB,
                                                              int64_t splitsB) {
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < nA + nB;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    const bool a = e < nA;
    const float* ws = a ? wsA : wsB;
    const int64_t n = a ? nA : nB, i = a ? e : e - nA, splits = a ? splitsA : splitsB;
    float s = 0.f;
    for (int64_t k = 0; k < splits; ++k) s += ws[k * n + i];
    Io<T>::store(a ? outA : outB, i, s);
  }
}

__global__ __launch_bounds__(256) void zero_kernel(uint16_t* p, int64_t n) {
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * 256)
    p[e] = 0;
}

inline int64_t iabs(int64_t v) { return v < 0 ? -v : v; }

}  // namespace

hipError_t launch_generic_gemm(const GemmArgs& a, bool bf16, hipStream_t s) {
  const int64_t mt = (a.M + BM - 1) / BM;
  const int64_t nt = (a.N + BN - 1) / BN;
  const int64_t grid = mt * nt * a.nblk * (a.partial ? a.splits : 1);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int a_k_fast = iabs(a.a_sk) <= iabs(a.a_si);
  const int b_k_fast = iabs(a.b_sk) <= iabs(a.b_sj);
  if (bf16)
    hipLaunchKernelGGL(generic_gemm_kernel<uint16_t>, dim3(static_cast<unsigned>(grid)), dim3(256),
                       0, s, a, mt, nt, a_k_fast, b_k_fast);
  else
    hipLaunchKernelGGL(generic_gemm_kernel<float>, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                       s, a, mt, nt, a_k_fast, b_k_fast);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(bytes / 2);
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<uint16_t*>(p), n);
  return hipGetLastError();
}

hipError_t launch_reduce_partials(const float* partialA, void* outA, int64_t nA, int64_t splitsA,
                                  const float* partialB, void* outB, int64_t nB, int64_t splitsB,
                                  bool bf16, hipStream_t s) {
  const int64_t n = nA + nB;
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (bf16)
    hipLaunchKernelGGL(reduce_partials_kernel<uint16_t>, dim3(static_cast<unsigned>(blocks)),
                       dim3(256), 0, s, partialA, outA, nA, splitsA, partialB, outB, nB, splitsB);
  else
    hipLaunchKernelGGL(reduce_partials_kernel<float>, dim3(static_cast<unsigned>(blocks)),
                       dim3(256), 0, s, partialA, outA, nA, splitsA, partialB, outB, nB, splitsB);
  return hipGetLastError();
}

}  // namespace monarch
