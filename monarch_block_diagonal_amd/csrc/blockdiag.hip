// Block-diagonal products with 256 x 256 weight blocks in bf16: the two
// block-sparse terms of the DYAD-style layer (DYAD page, abstract) once
// term B's operands are in block-major order, each multiplying nb
// independent 256-feature segments of a row by one dense block:
//   C[b, blk*cs + j] = sum_k A[b, blk*as + k] W_blk(k, j),   j, k < 256,
// with W_blk(k, j) = W[blk][j][k] (the forward: rows of the stored block are
// output features) or W[blk][k][j] (the data gradient: its transpose).
//
// At K = N = 256 a product moves 1 KB per row (512 bytes in, 512 out) for
// 64 Ki multiply-adds: 128 flop per byte, under the bf16 MFMA ridge of about
// 310 (2.5 PFLOP/s over 8 TB/s), so it is bound by HBM. The generic tiled GEMM covers it with 256 x 256
// tiles whose eight waves fill a CU's registers: a workgroup then loads,
// multiplies and stores in turn (4 K steps) with nothing to overlap.
// Here a workgroup owns one block and a row range:
//  * each of its eight waves keeps a 32-column slice of the weight block in
//    VGPRs (64 registers) for the whole launch;
//  * 32-row tiles of A pass through LDS (double-buffered, loaded one tile
//    ahead), results are staged in LDS and leave as whole 512-byte row
//    segments, one barrier per tile;
//  * 66 KB of LDS and at most 128 VGPRs per lane, so two workgroups share a
//    CU and one's loads overlap the other's stores;
//  * activations and results stream with non-temporal loads and stores
//    (each is touched once per launch, far beyond the L2).
// MFMA v_mfma_f32_16x16x32_bf16 computes Cᵀ[j x b] = Wᵀ-slice[j x k] · Aᵀ[k x b]
// with fp32 accumulation; each result is rounded once to bf16.
#include <stdint.h>

#include "common.h"
#include "kernels.h"

namespace monarch {
namespace {

constexpr int BQ = 256;           // block size (N = K)
constexpr int BT = 32;            // rows per tile
constexpr int BP = BQ + 8;        // LDS pitch (elements) of a [row][feature] tile
constexpr int kBdThreads = 512;

__device__ __forceinline__ bf16x8 bd_frag(const uint16_t* p) {
  return as_bf16x8(*reinterpret_cast<const u16x8*>(p));
}

template <bool TRANS>
__global__ __launch_bounds__(kBdThreads) __attribute__((amdgpu_waves_per_eu(4)))
void bd256_kernel(const uint16_t* __restrict__ A, int64_t a_sb, int64_t a_si,
                  const uint16_t* __restrict__ W, int64_t w_sb, uint16_t* __restrict__ C,
                  int64_t c_sb, int64_t c_si, int64_t rows, int64_t rows_per, int64_t nblk) {
  // [A tile 0][A tile 1][C tile 0][C tile 1]; in the prologue of the
  // transposed form, 64 rows of the weight block, transposed
  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * BT * BP];
  const int64_t blk = blockIdx.x % nblk;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x / nblk) * rows_per;
  const int64_t r1 = r0 + rows_per < rows ? r0 + rows_per : rows;
  if (r0 >= r1) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l15 = lane & 15, lh = lane >> 4;

  // MFMA A operand: lane holds W_blk(k = 32ks + 8lh .. +7, j = 32w + 16mt + l15)
  bf16x8 wf[2][8];
  const uint16_t* Wb = W + blk * w_sb;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int j = 32 * w + 16 * mt + l15;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int k = 32 * ks + 8 * lh;
      if constexpr (!TRANS) wf[mt][ks] = bd_frag(Wb + j * BQ + k);
    }
  }
  if constexpr (TRANS) {
    // W_blk(k, j) = W[blk][k][j]: k runs across rows of the stored block.
    // Four passes of 64 rows: 16-byte loads (lane = row, wave = 8-column
    // group, so the 2-byte stores of a wave hit 64 consecutive halfwords)
    // stored transposed into LDS as [j][64 k] (pitch 72), from which each
    // lane reads its fragments as 16-byte pieces.
    constexpr int TP = 64 + 8;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      u32x4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = tid + kBdThreads * i, kl = p & 63, j0 = (p >> 6) * 8;
        v[i] = *reinterpret_cast<const u32x4*>(Wb + (64 * h + kl) * BQ + j0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = tid + kBdThreads * i, kl = p & 63, j0 = (p >> 6) * 8;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          lds[(j0 + 2 * q) * TP + kl] = static_cast<uint16_t>(v[i][q] & 0xffffu);
          lds[(j0 + 2 * q + 1) * TP + kl] = static_cast<uint16_t>(v[i][q] >> 16);
        }
      }
      __syncthreads();
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int j = 32 * w + 16 * mt + l15;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) wf[mt][2 * h + kk] = bd_frag(&lds[j * TP + 32 * kk + 8 * lh]);
      }
      __syncthreads();
    }
  }

  // tile pieces: thread moves pieces tid and tid + 512 of a 32 x 256 tile,
  // piece p = (row p / 32, features 8 * (p % 32) .. +7)
  const int prow = tid >> 5, pcol = (tid & 31) * 8;
  const uint16_t* Ab = A + blk * a_sb + pcol;
  uint16_t* Cb = C + blk * c_sb + pcol;
  const int64_t ntiles = (r1 - r0 + BT - 1) / BT;
  u32x4 pre[2];
  auto gload = [&](int64_t t) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int64_t row = r0 + t * BT + prow + 16 * i;
      row = row < r1 ? row : r1 - 1;
      pre[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Ab + row * a_si));
    }
  };
  auto lstore = [&](uint16_t* x) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<u32x4*>(&x[(prow + 16 * i) * BP + pcol]) = pre[i];
  };

  gload(0);
  lstore(lds);
  if (ntiles > 1) gload(1);
  __syncthreads();
  for (int64_t t = 0; t < ntiles; ++t) {
    const int s = static_cast<int>(t & 1);
    const uint16_t* x = lds + s * (BT * BP);
    f32x4 acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      bf16x8 fb[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) fb[nt] = bd_frag(&x[(16 * nt + l15) * BP + 32 * ks + 8 * lh]);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[mt][ks], fb[nt], acc[mt][nt], 0, 0, 0);
    }
    // lane holds C[b = 16nt + l15][j = 32w + 16mt + 4lh .. +3]
    uint16_t* y = lds + (2 + s) * (BT * BP);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const u32x2 v{pack_bf16x2(acc[mt][nt][0], acc[mt][nt][1]),
                      pack_bf16x2(acc[mt][nt][2], acc[mt][nt][3])};
        *reinterpret_cast<u32x2*>(&y[(16 * nt + l15) * BP + 32 * w + 16 * mt + 4 * lh]) = v;
      }
    if (t + 1 < ntiles) {
      lstore(lds + (1 - s) * (BT * BP));
      if (t + 2 < ntiles) gload(t + 2);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t row = r0 + t * BT + prow + 16 * i;
      if (row < r1)
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(&y[(prow + 16 * i) * BP + pcol]),
                                    reinterpret_cast<u32x4*>(Cb + row * c_si));
    }
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

int bd256_mode(const GemmArgs& a, bool bf16) {
  if (!bf16 || a.partial || a.accum || a.bias || a.relu || a.mask || a.nsplit > 0) return 0;
  if (a.k_lim >= 0 || a.n_lim >= 0 || a.c_cols >= 0) return 0;
  if (a.N != BQ || a.K != BQ || a.M <= 0 || a.nblk <= 0) return 0;
  if (a.a_sk != 1 || a.c_sj != 1) return 0;
  if (a.a_si % 8 || a.a_sb % 8 || a.c_si % 8 || a.c_sb % 8) return 0;
  if (a.a_si <= 0 || a.c_si <= 0 || a.a_sb < 0 || a.c_sb < 0 || a.b_sb < 0) return 0;
  if (!aligned16(a.A) || !aligned16(a.C)) return 0;
  if (!aligned16(a.B) || a.b_sb % 8) return 0;
  if (a.b_sk == 1 && a.b_sj == BQ) return 1;
  if (a.b_sk == BQ && a.b_sj == 1) return 2;
  return 0;
}

hipError_t launch_bd256(const GemmArgs& a, int mode, hipStream_t s) {
  // about two workgroups per CU over the 256 CUs, each at least 4 tiles
  const int64_t tiles = (a.M + BT - 1) / BT;
  int64_t ranges = (512 + a.nblk - 1) / a.nblk;
  const int64_t rmax = (tiles + 3) / 4;
  if (ranges > rmax) ranges = rmax;
  if (ranges < 1) ranges = 1;
  const int64_t rows_per = (tiles + ranges - 1) / ranges * BT;
  ranges = (a.M + rows_per - 1) / rows_per;
  const int64_t grid = ranges * a.nblk;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const auto* A = static_cast<const uint16_t*>(a.A);
  const auto* W = static_cast<const uint16_t*>(a.B);
  auto* C = static_cast<uint16_t*>(a.C);
  if (mode == 1)
    bd256_kernel<false><<<dim3(static_cast<unsigned>(grid)), dim3(kBdThreads), 0, s>>>(
        A, a.a_sb, a.a_si, W, a.b_sb, C, a.c_sb, a.c_si, a.M, rows_per, a.nblk);
  else
    bd256_kernel<true><<<dim3(static_cast<unsigned>(grid)), dim3(kBdThreads), 0, s>>>(
        A, a.a_sb, a.a_si, W, a.b_sb, C, a.c_sb, a.c_si, a.M, rows_per, a.nblk);
  return hipGetLastError();
}

}  // namespace monarch
