// Block-diagonal products in bf16 whose weight blocks fit a CU's registers
// when split into 256-column slices, with K = 192 or 256 per block:
//   C[b, blk*cs + col(j)] = sum_k A[b, blk*as + k] W_blk(k, j),   k < K,
// with W_blk(k, j) = W[blk][row(j)][k] (rows of the stored block are output
// features) or, for 256 x 256 blocks only, W[blk][k][j] (the data gradient:
// its transpose). row(j) and col(j) follow the optional column split of
// GemmArgs: the stage-1 forward of a Monarch layer (Definition C.3 thread of
// the scatterbrain issues page) stores block r's output k = tt*b2 + g at
// stage 2's position g*q2i + r*n1 + tt, so its weight rows are gathered in
// that order and its outputs leave as runs of n1 columns. Two users:
//  * the two block-sparse terms of the DYAD-style layer (DYAD page,
//    abstract), 256 x 256 blocks once term B's operands are block-major;
//  * the stage-1 forward of Monarch layers with q1i = 192 or 256 and q1o a
//    multiple of 256, e.g. the GPT-2 FFN up-projection 768 -> 3072 with 4
//    blocks (768 x 192 blocks, taken as three 256-column slices).
//
// A product moves (K + N) * 2 bytes per row for K * N multiply-adds: at
// K = 192..256 that is 96..128 flop per byte, under the bf16 MFMA ridge of
// about 310 (2.5 PFLOP/s over 8 TB/s), so it is bound by HBM. The generic
// tiled GEMM covers it with 256 x 256 tiles whose eight waves fill a CU's
// registers: a workgroup then loads, multiplies and stores in turn (6 or 8
// K steps) with nothing to overlap. Here a workgroup owns one block, one
// 256-column slice of it and a row range:
//  * each of its eight waves keeps a 32-column piece of the slice in VGPRs
//    (K/4 registers) for the whole launch;
//  * 32-row tiles of A pass through LDS (double-buffered, loaded one tile
//    ahead), results are staged in LDS and leave as 16-byte pieces of whole
//    512-byte row segments (or of the split's runs), one barrier per tile;
//  * at most 66 KB of LDS and 128 VGPRs per lane, so two workgroups share a
//    CU and one's loads overlap the other's stores;
//  * the slices of one block read the same A rows: they are given
//    consecutive ids on one XCD, so those rows come from HBM once;
//  * activations and results stream with non-temporal loads and stores
//    (each is touched once per launch, far beyond the L2).
// MFMA v_mfma_f32_16x16x32_bf16 computes Cᵀ[j x b] = Wᵀ-slice[j x k] · Aᵀ[k x b]
// with fp32 accumulation; each result is rounded once to bf16.
#include <stdint.h>

#include <numeric>

#include "common.h"
#include "kernels.h"

namespace monarch {
namespace {

constexpr int BQ = 256;           // columns per slice; block size of the transposed form
constexpr int BT = 32;            // rows per tile
constexpr int BP = BQ + 8;        // LDS pitch (elements) of a [row][column] result tile
constexpr int kBdThreads = 512;

__device__ __forceinline__ bf16x8 bd_frag(const uint16_t* p) {
  return as_bf16x8(*reinterpret_cast<const u16x8*>(p));
}

// Column offsets under the optional split (GemmArgs): j*lo, or
// (j / ns)*hi + (j % ns)*lo when ns > 0.
struct Split {
  int64_t ns, hi, lo;
  __device__ __forceinline__ int64_t operator()(int64_t j) const {
    return ns > 0 ? (j / ns) * hi + (j % ns) * lo : j * lo;
  }
};

template <bool TRANS, int KB>
__global__ __launch_bounds__(kBdThreads) __attribute__((amdgpu_waves_per_eu(4)))
void bd_kernel(const uint16_t* __restrict__ A, int64_t a_sb, int64_t a_si,
               const uint16_t* __restrict__ W, int64_t w_sb, Split wrow,
               uint16_t* __restrict__ C, int64_t c_sb, int64_t c_si, Split ccol,
               int64_t rows, int64_t rows_per, int64_t nblk, int nslices, int remap) {
  static_assert(KB == 192 || KB == 256, "K per block");
  static_assert(!TRANS || KB == BQ, "the transposed form takes 256 x 256 blocks");
  constexpr int KP = KB + 8;               // LDS pitch of a [row][k] operand tile
  constexpr int KS = KB / 32;              // MFMA K steps
  constexpr int APR = KB / 8;              // 16-byte pieces per operand row
  constexpr int NA = (BT * APR + kBdThreads - 1) / kBdThreads;   // pieces per thread
  // [A tile 0][A tile 1][C tile 0][C tile 1]; in the prologue of the
  // transposed form, 64 rows of the weight block, transposed
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * BT * KP + 2 * BT * BP];
  int64_t logical = blockIdx.x;
  if (remap) logical = (logical & 7) * (gridDim.x >> 3) + (logical >> 3);
  const int64_t blk = logical % nblk;
  const int64_t rest = logical / nblk;
  const int64_t j0 = (rest % nslices) * BQ;
  const int64_t r0 = (rest / nslices) * rows_per;
  const int64_t r1 = r0 + rows_per < rows ? r0 + rows_per : rows;
  if (r0 >= r1) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l15 = lane & 15, lh = lane >> 4;

  // MFMA A operand: lane holds W_blk(k = 32ks + 8lh .. +7, j = j0 + 32w + 16mt + l15)
  bf16x8 wf[2][KS];
  const uint16_t* Wb = W + blk * w_sb;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int64_t jr = wrow(j0 + 32 * w + 16 * mt + l15);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int k = 32 * ks + 8 * lh;
      if constexpr (!TRANS) wf[mt][ks] = bd_frag(Wb + jr + k);
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
        const int p = tid + kBdThreads * i, kl = p & 63, jg = (p >> 6) * 8;
        v[i] = *reinterpret_cast<const u32x4*>(Wb + (64 * h + kl) * BQ + jg);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = tid + kBdThreads * i, kl = p & 63, jg = (p >> 6) * 8;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          lds[(jg + 2 * q) * TP + kl] = static_cast<uint16_t>(v[i][q] & 0xffffu);
          lds[(jg + 2 * q + 1) * TP + kl] = static_cast<uint16_t>(v[i][q] >> 16);
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

  // operand pieces: thread moves pieces tid + 512i of a 32 x KB tile, piece
  // p = (row p / APR, k 8 * (p % APR) .. +7); result pieces: tid and tid +
  // 512 of a 32 x 256 tile, piece (row tid / 32 + 16i, columns 8 * (tid % 32) .. +7)
  int arow[NA], acol[NA];
  bool aon[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int pc = tid + kBdThreads * i;
    // every piece is real when the tile divides evenly (K = 256)
    aon[i] = (BT * APR) % kBdThreads == 0 || pc < BT * APR;
    arow[i] = aon[i] ? pc / APR : 0;
    acol[i] = aon[i] ? (pc % APR) * 8 : 0;
  }
  const int prow = tid >> 5, pcol = (tid & 31) * 8;
  const uint16_t* Ab = A + blk * a_sb;
  // the 8 columns of a result piece lie in one run of the split
  uint16_t* Cb = C + blk * c_sb + ccol(j0 + pcol);
  const int64_t ntiles = (r1 - r0 + BT - 1) / BT;
  u32x4 pre[NA];
  auto gload = [&](int64_t t) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      if (!aon[i]) continue;
      int64_t row = r0 + t * BT + arow[i];
      row = row < r1 ? row : r1 - 1;
      pre[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Ab + row * a_si + acol[i]));
    }
  };
  auto lstore = [&](uint16_t* x) {
#pragma unroll
    for (int i = 0; i < NA; ++i)
      if (aon[i]) *reinterpret_cast<u32x4*>(&x[arow[i] * KP + acol[i]]) = pre[i];
  };
  uint16_t* const cst = lds + 2 * BT * KP;   // result tiles

  gload(0);
  lstore(lds);
  if (ntiles > 1) gload(1);
  __syncthreads();
  for (int64_t t = 0; t < ntiles; ++t) {
    const int s = static_cast<int>(t & 1);
    const uint16_t* x = lds + s * (BT * KP);
    f32x4 acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 fb[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) fb[nt] = bd_frag(&x[(16 * nt + l15) * KP + 32 * ks + 8 * lh]);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[mt][ks], fb[nt], acc[mt][nt], 0, 0, 0);
    }
    // lane holds C[b = 16nt + l15][j = j0 + 32w + 16mt + 4lh .. +3]
    uint16_t* y = cst + s * (BT * BP);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const u32x2 v{pack_bf16x2(acc[mt][nt][0], acc[mt][nt][1]),
                      pack_bf16x2(acc[mt][nt][2], acc[mt][nt][3])};
        *reinterpret_cast<u32x2*>(&y[(16 * nt + l15) * BP + 32 * w + 16 * mt + 4 * lh]) = v;
      }
    if (t + 1 < ntiles) {
      lstore(lds + (1 - s) * (BT * KP));
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

int bd_mode(const GemmArgs& a, bool bf16) {
  if (!bf16 || a.partial || a.accum || a.bias || a.relu || a.mask) return 0;
  if (a.n_lim >= 0 || a.c_cols >= 0) return 0;
  if (a.M <= 0 || a.nblk <= 0 || a.N <= 0 || a.N % BQ || (a.K != 192 && a.K != BQ)) return 0;
  // zero padding is allowed when it cuts no block
  if (a.k_lim >= 0 && a.k_lim - (a.nblk - 1) * a.k_lim_bs < a.K) return 0;
  if (a.a_sk != 1 || a.c_sj != 1) return 0;
  if (a.a_si % 8 || a.a_sb % 8 || a.c_si % 8 || a.c_sb % 8) return 0;
  if (a.a_si <= 0 || a.c_si <= 0 || a.a_sb < 0 || a.c_sb < 0 || a.b_sb < 0) return 0;
  if (!aligned16(a.A) || !aligned16(a.C)) return 0;
  if (!aligned16(a.B) || a.b_sb % 8) return 0;
  // a split keeps every 8-column piece (weights and results) in one run
  if (a.nsplit > 0 && (a.nsplit % 8 || a.b_sj_hi < 0 || a.b_sj_hi % 8 || a.c_sj_hi < 0 ||
                       a.c_sj_hi % 8))
    return 0;
  if (a.b_sk == 1 && a.b_sj > 0 && a.b_sj % 8 == 0) return a.K == BQ ? 1 : 3;
  if (a.nsplit == 0 && a.K == BQ && a.N == BQ && a.b_sk == BQ && a.b_sj == 1) return 2;
  return 0;
}

hipError_t launch_bd(const GemmArgs& a, int mode, hipStream_t s) {
  // about two workgroups per CU over the 256 CUs, each at least 4 tiles
  const int64_t nslices = a.N / BQ;
  const int64_t per_range = a.nblk * nslices;
  const int64_t tiles = (a.M + BT - 1) / BT;
  int64_t ranges = (512 + per_range - 1) / per_range;
  const int64_t rmax = (tiles + 3) / 4;
  if (ranges > rmax) ranges = rmax;
  if (ranges < 1) ranges = 1;
  // the slices of a block share their A rows: consecutive ids go to one XCD
  // (workgroups are dispatched round-robin over the 8 XCDs), which needs a
  // grid that is a multiple of 8; workgroups of trailing empty ranges exit
  const int remap = nslices > 1 ? 1 : 0;
  if (remap) {
    const int64_t q = 8 / std::gcd(per_range, int64_t(8));
    ranges = (ranges + q - 1) / q * q;
  }
  const int64_t rows_per = (tiles + ranges - 1) / ranges * BT;
  if (!remap) ranges = (a.M + rows_per - 1) / rows_per;
  const int64_t grid = ranges * per_range;
  if (grid > 0x7fffffffLL || nslices > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const auto* A = static_cast<const uint16_t*>(a.A);
  const auto* W = static_cast<const uint16_t*>(a.B);
  auto* C = static_cast<uint16_t*>(a.C);
  const Split wrow{a.nsplit, a.b_sj_hi, a.b_sj}, ccol{a.nsplit, a.c_sj_hi, 1};
  const dim3 g(static_cast<unsigned>(grid)), blk(kBdThreads);
  const int ns = static_cast<int>(nslices);
  switch (mode) {
    case 1:
      bd_kernel<false, 256><<<g, blk, 0, s>>>(A, a.a_sb, a.a_si, W, a.b_sb, wrow, C, a.c_sb,
                                               a.c_si, ccol, a.M, rows_per, a.nblk, ns, remap);
      break;
    case 2:
      bd_kernel<true, 256><<<g, blk, 0, s>>>(A, a.a_sb, a.a_si, W, a.b_sb, wrow, C, a.c_sb,
                                              a.c_si, ccol, a.M, rows_per, a.nblk, ns, remap);
      break;
    case 3:
      bd_kernel<false, 192><<<g, blk, 0, s>>>(A, a.a_sb, a.a_si, W, a.b_sb, wrow, C, a.c_sb,
                                               a.c_si, ccol, a.M, rows_per, a.nblk, ns, remap);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace monarch
