// Fast path for bf16 Monarch layers whose four block dimensions are all 128
// (in = mid = out = 128*b, nblocks1 = nblocks2 = b, b a multiple of 8): the
// square Definition C.3 family (scatterbrain issues page, "Definition C.3"
// thread) at block size 128, e.g. n = 16384 with 128 blocks.
//
// At this block size every stage is HBM-bound (64 flop per byte moved at the
// I/O width against a bf16 MFMA ridge near 300), so the kernels are built
// around data movement:
//
//  * The saved stage-2 input Z (and the backward's dZ) use a panel layout:
//    feature j of row b sits at ((j/8)*B + b)*8 + j%8. A stage-1 kernel that
//    owns one R block writes 16 whole panels (256-512 B runs); a stage-2
//    kernel that owns 8 consecutive L blocks g0..g0+7 finds, for each t, its
//    8 inputs Z[b, t*b2 + g0 .. +7] in one panel (the stride permutation of
//    the "hypercube" thread becomes a panel index, no permuted copy exists).
//  * The caller's row-major Y / dY put the 8 L blocks of a workgroup in one
//    16-byte run per (row, p). The stage-2 workgroups that share those cache
//    lines are mapped onto one XCD (workgroups are dispatched round-robin
//    over the 8 XCDs) so partial lines merge in that XCD's L2.
//  * Weights stay in VGPRs for the whole launch (persistent workgroups over
//    a row range); MFMA v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
//  * Weight gradients accumulate in registers over a batch chunk per
//    workgroup; chunks are summed afterwards in a fixed order.
#include "common.h"
#include "square.h"

namespace monarch {
namespace {

constexpr int Q = 128;        // block size
constexpr int XLD = Q + 8;    // LDS pitch (elements) of [row][feature] tiles
constexpr int TLD = 32 + 8;   // LDS pitch of [feature][32 rows] tiles
constexpr int YLD = Q * 8 + 8;

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void stg16(uint16_t* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ bf16x8 frag_ld(const uint16_t* p) {
  return as_bf16x8(*reinterpret_cast<const u16x8*>(p));
}
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint16_t half_of(u32x4 v, int e) {
  const uint32_t w = v[e >> 1];
  return static_cast<uint16_t>((e & 1) ? (w >> 16) : (w & 0xffffu));
}
// bf16 bit pattern strictly greater than zero (NaN excluded)
__device__ __forceinline__ bool bf16_pos(uint32_t h) {
  return (h & 0x8000u) == 0 && (h & 0x7fffu) != 0 && (h & 0x7fffu) <= 0x7f80u;
}
// zero the halves of v whose mask half is not > 0 (ReLU derivative)
__device__ __forceinline__ u32x4 apply_mask(u32x4 v, u32x4 m) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t keep = (bf16_pos(m[i] & 0xffffu) ? 0xffffu : 0u) |
                    (bf16_pos(m[i] >> 16) ? 0xffff0000u : 0u);
    r[i] = v[i] & keep;
  }
  return r;
}
// workgroups are dispatched round-robin over the 8 XCDs: give consecutive
// logical ids to one XCD
__device__ __forceinline__ int xcd_logical(int bid, int grid) {
  if (grid & 7) return bid;
  return (bid & 7) * (grid >> 3) + (bid >> 3);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Conventions of the kernels below.
//  * Element offsets are 32-bit, relative to a per-tile base pointer;
//    sq_applicable() admits only problems with batch*features < 2^31.
//  * Every load and store in a main loop is unconditional, so the compiler
//    can count outstanding memory operations exactly and keep two prefetched
//    tiles in flight. Rows past the end of a workgroup's range are clamped to
//    its last row: duplicated outputs are recomputed from the same inputs and
//    store identical values to the same address, and rows that feed a
//    weight-gradient sum are zeroed instead.
//  * A workgroup walks its row range in pairs of tiles (slots A and B); a
//    trailing odd tile is a clamped duplicate.

// Wait once for everything the prologue issued (weights and the first two
// tiles). The wait counts the compiler inserts at a loop head are the
// minimum over its predecessors; without this, the prologue's issue order
// would set them and drain both prefetch slots on every iteration.
__device__ __forceinline__ void drain_prologue() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ int clamp_row(int row, int64_t lim) {
  return row < lim ? row : static_cast<int>(lim - 1);
}
__device__ __forceinline__ u32x4 zero_unless(bool keep, u32x4 v) {
  return keep ? v : u32x4{0u, 0u, 0u, 0u};
}

// --------------------------------------------------------------------------
// stage 1 forward: Z_r = X_r · R_rᵀ for one R block per workgroup
// --------------------------------------------------------------------------
// 4 waves; wave w owns output features k in [32w, 32w+32). Tile: 32 rows.
// C = Zᵀ[k x b] = R[k x s] · Xᵀ[s x b]; A = R fragments in VGPRs, B = X tile
// from LDS; results go straight to the panel layout (lane pairs fill 16 B,
// 16 lanes fill 256 B of one panel).
__global__ __launch_bounds__(256) void sq_stage1_fwd_kernel(const uint16_t* __restrict__ X,
                                                            const uint16_t* __restrict__ W1,
                                                            uint16_t* __restrict__ Z, int64_t B,
                                                            int nb1, int64_t rows_per) {
  constexpr int T = 32;
  __shared__ __attribute__((aligned(16))) uint16_t xs[T * XLD];
  const int r = blockIdx.x % nb1;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x / nb1) * rows_per;
  const int64_t row1 = row0 + rows_per < B ? row0 + rows_per : B;
  if (row0 >= row1) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l15 = lane & 15, lh = lane >> 4;
  const uint32_t in = static_cast<uint32_t>(nb1) * Q;
  const uint32_t Bu = static_cast<uint32_t>(B);

  bf16x8 a[2][4];
  const uint16_t* Rr = W1 + static_cast<int64_t>(r) * Q * Q;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      a[mt][ks] = frag_ld(Rr + (32 * w + 16 * mt + l15) * Q + 32 * ks + 8 * lh);

  // X pieces: row = (tid>>4) + 16i, seg = tid&15
  const int lrow = tid >> 4, seg = tid & 15;
  const uint32_t xcol = r * Q + seg * 8;
  // Z stores: panel r*16 + 4w + 2mt + lh/2, row 16nt + l15
  const uint32_t zcol = (r * 16 + 4 * w + (lh >> 1)) * Bu * 8 + 4 * (lh & 1);

  auto gload = [&](u32x4(&pre)[2], int64_t b0) {
    const int64_t bc = b0 < row1 ? b0 : row1 - 1, lim = row1 - bc;
    const uint16_t* base = X + bc * in;
#pragma unroll
    for (int i = 0; i < 2; ++i) pre[i] = ldg16(base + clamp_row(lrow + 16 * i, lim) * in + xcol);
  };
  auto body = [&](u32x4(&cur)[2], int64_t b0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4*>(&xs[(lrow + 16 * i) * XLD + seg * 8]) = cur[i];
    __syncthreads();
    gload(cur, b0 + 2 * T);
    f32x4 acc[2][2] = {{zero4(), zero4()}, {zero4(), zero4()}};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 bop[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) bop[nt] = frag_ld(&xs[(16 * nt + l15) * XLD + 32 * ks + 8 * lh]);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma(a[mt][ks], bop[nt], acc[mt][nt]);
    }
    const int64_t bc = b0 < row1 ? b0 : row1 - 1, lim = row1 - bc;
    uint16_t* zb = Z + bc * 8;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        u32x2 v;
        v[0] = pack_bf16x2(acc[mt][nt][0], acc[mt][nt][1]);
        v[1] = pack_bf16x2(acc[mt][nt][2], acc[mt][nt][3]);
        *reinterpret_cast<u32x2*>(zb + zcol + 2 * mt * Bu * 8 + clamp_row(16 * nt + l15, lim) * 8) = v;
      }
    __syncthreads();
  };

  const int64_t npairs = (row1 - row0 + 2 * T - 1) / (2 * T);
  u32x4 pa[2], pb[2];
  gload(pa, row0);
  gload(pb, row0 + T);
  drain_prologue();
  for (int64_t k = 0; k < npairs; ++k) {
    body(pa, row0 + 2 * k * T);
    body(pb, row0 + (2 * k + 1) * T);
  }
}

// --------------------------------------------------------------------------
// stage 2 forward: Y[b, p*b2 + g] = act(sum_t L[g,p,t] Z[b, t*b2 + g])
// --------------------------------------------------------------------------
// 8 waves, 8 L blocks g0..g0+7 per workgroup; wave w owns block g0 + w with
// all of L_g in VGPRs. Tile: 16 rows; two tiles of Z panels are in flight in
// registers while a third is computed. Z panels -> LDS [g][row][t];
// C = Vᵀ[p x b] = L[p x t] · Wᵀ[t x b]; results -> LDS [row][p][g] -> Y in
// 16-byte runs.
__global__ __launch_bounds__(512) void sq_stage2_fwd_kernel(const uint16_t* __restrict__ Z,
                                                            const uint16_t* __restrict__ W2,
                                                            uint16_t* __restrict__ Y, int64_t B,
                                                            int nb2, int64_t rows_per, int relu) {
  constexpr int T = 16;
  __shared__ __attribute__((aligned(16))) uint16_t ws[8 * T * XLD];
  __shared__ __attribute__((aligned(16))) uint16_t ys[T * YLD];
  const int n_groups = nb2 >> 3;
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int gg = logical % n_groups;
  const int64_t row0 = static_cast<int64_t>(logical / n_groups) * rows_per;
  const int64_t row1 = row0 + rows_per < B ? row0 + rows_per : B;
  if (row0 >= row1) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l15 = lane & 15, lh = lane >> 4;
  const int g = gg * 8 + w;
  const uint32_t out = static_cast<uint32_t>(nb2) * Q;
  const uint32_t Bu = static_cast<uint32_t>(B);
  const uint32_t pstride = nb2 >> 3;  // panels between t and t+1

  bf16x8 a[8][4];
  const uint16_t* Lg = W2 + static_cast<int64_t>(g) * Q * Q;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a[mt][ks] = frag_ld(Lg + (16 * mt + l15) * Q + 32 * ks + 8 * lh);

  // Z pieces: t = (tid>>4) + 32i, row = tid&15; Y pieces: row = (tid>>7) + 4i, p = tid&127
  const int zt = tid >> 4, zrow = tid & 15;
  const uint32_t zcol = (zt * pstride + gg) * Bu * 8;
  const uint32_t zstep = 32 * pstride * Bu * 8;
  const int yrow = tid >> 7, yp = tid & 127;
  const uint32_t ycol = yp * nb2 + gg * 8;

  auto gload = [&](u32x4(&pre)[4], int64_t b0) {
    const int64_t bc = b0 < row1 ? b0 : row1 - 1, lim = row1 - bc;
    const uint16_t* base = Z + bc * 8 + clamp_row(zrow, lim) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) pre[i] = ldg16(base + zcol + i * zstep);
  };
  auto body = [&](u32x4(&cur)[4], int64_t b0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) ws[(e * T + zrow) * XLD + zt + 32 * i] = half_of(cur[i], e);
    __syncthreads();
    gload(cur, b0 + 2 * T);
    f32x4 acc[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[mt] = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 bop = frag_ld(&ws[(w * T + l15) * XLD + 32 * ks + 8 * lh]);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) acc[mt] = mfma(a[mt][ks], bop, acc[mt]);
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int v = 0; v < 4; v += 2) {
        float v0 = acc[mt][v], v1 = acc[mt][v + 1];
        if (relu) {
          v0 = v0 > 0.f ? v0 : 0.f;
          v1 = v1 > 0.f ? v1 : 0.f;
        }
        const uint32_t pk = pack_bf16x2(v0, v1);
        ys[l15 * YLD + (16 * mt + 4 * lh + v) * 8 + w] = static_cast<uint16_t>(pk & 0xffffu);
        ys[l15 * YLD + (16 * mt + 4 * lh + v + 1) * 8 + w] = static_cast<uint16_t>(pk >> 16);
      }
    __syncthreads();
    const int64_t bc = b0 < row1 ? b0 : row1 - 1, lim = row1 - bc;
    uint16_t* yb = Y + bc * out + ycol;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      stg16(yb + clamp_row(yrow + 4 * i, lim) * out,
            *reinterpret_cast<const u32x4*>(&ys[(yrow + 4 * i) * YLD + yp * 8]));
  };

  const int64_t npairs = (row1 - row0 + 2 * T - 1) / (2 * T);
  u32x4 pa[4], pb[4];
  gload(pa, row0);
  gload(pb, row0 + T);
  drain_prologue();
  for (int64_t k = 0; k < npairs; ++k) {
    body(pa, row0 + 2 * k * T);
    body(pb, row0 + (2 * k + 1) * T);
  }
}

// --------------------------------------------------------------------------
// stage 2 backward, data: dZ[b, t*b2 + g] = sum_p dYe[b, p*b2 + g] L[g,p,t]
// --------------------------------------------------------------------------
// Same tiling and pipeline as the forward; wave w owns block g0 + w.
// dY (masked) -> LDS [g][row][p]; C = dZᵀ[t x b] = Lᵀ[t x p] · dVᵀ[p x b];
// results -> LDS [t][row][g] -> dZ panels (256 B per t). The ReLU mask is
// read when a tile is consumed, not prefetched.
template <bool MASK>
__global__ __launch_bounds__(512) void sq_stage2_bwd_data_kernel(
    const uint16_t* __restrict__ dY, const uint16_t* __restrict__ Ym,
    const uint16_t* __restrict__ W2t, uint16_t* __restrict__ dZ, int64_t B, int nb2,
    int64_t rows_per) {
  constexpr int T = 16;
  __shared__ __attribute__((aligned(16))) uint16_t dvs[8 * T * XLD];
  __shared__ __attribute__((aligned(16))) uint16_t zs[Q * XLD];
  const int n_groups = nb2 >> 3;
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int gg = logical % n_groups;
  const int64_t row0 = static_cast<int64_t>(logical / n_groups) * rows_per;
  const int64_t row1 = row0 + rows_per < B ? row0 + rows_per : B;
  if (row0 >= row1) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l15 = lane & 15, lh = lane >> 4;
  const int g = gg * 8 + w;
  const uint32_t out = static_cast<uint32_t>(nb2) * Q;
  const uint32_t Bu = static_cast<uint32_t>(B);
  const uint32_t pstride = nb2 >> 3;

  // A = Lᵀ[t x p] from the transposed copy: lane holds L[g][p = 32ks + 8lh + e][t = 16mt + l15]
  bf16x8 a[8][4];
  const uint16_t* Ltg = W2t + static_cast<int64_t>(g) * Q * Q;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a[mt][ks] = frag_ld(Ltg + (16 * mt + l15) * Q + 32 * ks + 8 * lh);

  // dY pieces: row = (tid>>7) + 4i, p = tid&127; dZ pieces: t = (tid>>4) + 32i, row = tid&15
  const int drow = tid >> 7, dp = tid & 127;
  const uint32_t dcol = dp * nb2 + gg * 8;
  const int zt = tid >> 4, zrow = tid & 15;
  const uint32_t zcol = (zt * pstride + gg) * Bu * 8;
  const uint32_t zstep = 32 * pstride * Bu * 8;

  auto gload = [&](u32x4(&pre)[4], int64_t b0) {
    const int64_t bc = b0 < row1 ? b0 : row1 - 1, lim = row1 - bc;
    const uint16_t* base = dY + bc * out + dcol;
#pragma unroll
    for (int i = 0; i < 4; ++i) pre[i] = ldg16(base + clamp_row(drow + 4 * i, lim) * out);
  };
  auto body = [&](u32x4(&cur)[4], int64_t b0) {
    if constexpr (MASK) {
      const int64_t bc = b0 < row1 ? b0 : row1 - 1, lim = row1 - bc;
      const uint16_t* mb = Ym + bc * out + dcol;
#pragma unroll
      for (int i = 0; i < 4; ++i) cur[i] = apply_mask(cur[i], ldg16(mb + clamp_row(drow + 4 * i, lim) * out));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) dvs[(e * T + drow + 4 * i) * XLD + dp] = half_of(cur[i], e);
    __syncthreads();
    gload(cur, b0 + 2 * T);
    f32x4 acc[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[mt] = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 bop = frag_ld(&dvs[(w * T + l15) * XLD + 32 * ks + 8 * lh]);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) acc[mt] = mfma(a[mt][ks], bop, acc[mt]);
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int v = 0; v < 4; v += 2) {
        const uint32_t pk = pack_bf16x2(acc[mt][v], acc[mt][v + 1]);
        zs[(16 * mt + 4 * lh + v) * XLD + l15 * 8 + w] = static_cast<uint16_t>(pk & 0xffffu);
        zs[(16 * mt + 4 * lh + v + 1) * XLD + l15 * 8 + w] = static_cast<uint16_t>(pk >> 16);
      }
    __syncthreads();
    const int64_t bc = b0 < row1 ? b0 : row1 - 1, lim = row1 - bc;
    uint16_t* zb = dZ + bc * 8 + clamp_row(zrow, lim) * 8 + zcol;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      stg16(zb + i * zstep, *reinterpret_cast<const u32x4*>(&zs[(zt + 32 * i) * XLD + zrow * 8]));
  };

  const int64_t npairs = (row1 - row0 + 2 * T - 1) / (2 * T);
  u32x4 pa[4], pb[4];
  gload(pa, row0);
  gload(pb, row0 + T);
  drain_prologue();
  for (int64_t k = 0; k < npairs; ++k) {
    body(pa, row0 + 2 * k * T);
    body(pb, row0 + (2 * k + 1) * T);
  }
}

// --------------------------------------------------------------------------
// stage 2 backward, weights: dL[g,p,t] = sum_b dYe[b, p*b2+g] Z[b, t*b2+g]
// --------------------------------------------------------------------------
// Workgroup: 8 L blocks x a 32-wide slice of p x a batch chunk. 8 waves;
// wave w owns block g0 + w, accumulators dL[32 p x 128 t] in VGPRs. Tile: 32
// rows = one K step; two tiles in flight in registers. dY slice -> LDS
// [g][p][row], Z panels -> LDS [g][t][row] (row-contiguous operands for
// K = batch). Rows past the range enter as zero dY. The chunk's sum is
// written as an fp32 partial.
template <bool MASK>
__global__ __launch_bounds__(512) void sq_stage2_bwd_weight_kernel(
    const uint16_t* __restrict__ dY, const uint16_t* __restrict__ Ym,
    const uint16_t* __restrict__ Z, float* __restrict__ partial, int64_t B, int nb2,
    int64_t rows_per) {
  constexpr int T = 32;
  __shared__ __attribute__((aligned(16))) uint16_t dvs[8 * 32 * TLD];
  __shared__ __attribute__((aligned(16))) uint16_t zst[8 * Q * TLD];
  const int n_groups = nb2 >> 3;
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int ps = logical & 3;
  const int gg = (logical >> 2) % n_groups;
  const int chunk = (logical >> 2) / n_groups;
  const int64_t row0 = static_cast<int64_t>(chunk) * rows_per;
  const int64_t row1 = row0 + rows_per < B ? row0 + rows_per : B;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l15 = lane & 15, lh = lane >> 4;
  const int g = gg * 8 + w;
  const uint32_t out = static_cast<uint32_t>(nb2) * Q;
  const uint32_t Bu = static_cast<uint32_t>(B);
  const uint32_t pstride = nb2 >> 3;

  f32x4 acc[2][8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = zero4();

  // dY slice: row = (tid>>5) + 16i, pl = tid&31 (i < 2); Z: t = (tid>>5) + 16i, row = tid&31 (i < 8)
  const int hi = tid >> 5, lo = tid & 31;
  const uint32_t dcol = (32 * ps + lo) * nb2 + gg * 8;
  const uint32_t zcol = (hi * pstride + gg) * Bu * 8;
  const uint32_t zstep = 16 * pstride * Bu * 8;

  auto gload = [&](u32x4(&pd)[2], u32x4(&pz)[8], int64_t b0) {
    const int64_t bc = b0 < row1 ? b0 : row1 - 1, lim = row1 - bc;
    const uint16_t* db = dY + bc * out + dcol;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      pd[i] = zero_unless(b0 + hi + 16 * i < row1, ldg16(db + clamp_row(hi + 16 * i, lim) * out));
    const uint16_t* zb = Z + bc * 8 + clamp_row(lo, lim) * 8 + zcol;
#pragma unroll
    for (int i = 0; i < 8; ++i) pz[i] = ldg16(zb + i * zstep);
  };
  auto body = [&](u32x4(&pd)[2], u32x4(&pz)[8], int64_t b0) {
    if constexpr (MASK) {
      const int64_t bc = b0 < row1 ? b0 : row1 - 1, lim = row1 - bc;
      const uint16_t* mb = Ym + bc * out + dcol;
#pragma unroll
      for (int i = 0; i < 2; ++i) pd[i] = apply_mask(pd[i], ldg16(mb + clamp_row(hi + 16 * i, lim) * out));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) dvs[(e * 32 + lo) * TLD + hi + 16 * i] = half_of(pd[i], e);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) zst[(e * Q + hi + 16 * i) * TLD + lo] = half_of(pz[i], e);
    __syncthreads();
    gload(pd, pz, b0 + 2 * T);
    bf16x8 A[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) A[mt] = frag_ld(&dvs[(w * 32 + 16 * mt + l15) * TLD + 8 * lh]);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const bf16x8 Bv = frag_ld(&zst[(w * Q + 16 * nt + l15) * TLD + 8 * lh]);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) acc[mt][nt] = mfma(A[mt], Bv, acc[mt][nt]);
    }
    __syncthreads();
  };

  if (row0 < row1) {
    const int64_t npairs = (row1 - row0 + 2 * T - 1) / (2 * T);
    u32x4 da[2], za[8], db[2], zb[8];
    gload(da, za, row0);
    gload(db, zb, row0 + T);
    drain_prologue();
    for (int64_t k = 0; k < npairs; ++k) {
      body(da, za, row0 + 2 * k * T);
      body(db, zb, row0 + (2 * k + 1) * T);
    }
  }
  // partial[chunk][g][p][t]
  float* P = partial + (static_cast<int64_t>(chunk) * nb2 + g) * Q * Q;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        P[(32 * ps + 16 * mt + 4 * lh + v) * Q + 16 * nt + l15] = acc[mt][nt][v];
}

// --------------------------------------------------------------------------
// stage 1 backward: dX_r = dZ_r · R_r and dR_r = sum_b dZ_rᵀ X_r
// --------------------------------------------------------------------------
// One R block and a batch chunk per workgroup, 8 waves; wave w owns dX
// features s in [16w, +16) and dR rows k in [16w, +16). Tile: 32 rows; two
// tiles in flight in registers. dZ panels -> LDS [row][k] and [k][row];
// X -> LDS [s][row] (zero past the range, so dR only sums real rows).
__global__ __launch_bounds__(512) void sq_stage1_bwd_kernel(
    const uint16_t* __restrict__ dZ, const uint16_t* __restrict__ X,
    const uint16_t* __restrict__ W1t, uint16_t* __restrict__ dX, float* __restrict__ partial,
    int64_t B, int nb1, int64_t rows_per) {
  constexpr int T = 32;
  __shared__ __attribute__((aligned(16))) uint16_t dzs[T * XLD];
  __shared__ __attribute__((aligned(16))) uint16_t dzt[Q * TLD];
  __shared__ __attribute__((aligned(16))) uint16_t xt[Q * TLD];
  __shared__ __attribute__((aligned(16))) uint16_t dxs[T * XLD];
  const int r = blockIdx.x % nb1;
  const int chunk = blockIdx.x / nb1;
  const int64_t row0 = static_cast<int64_t>(chunk) * rows_per;
  const int64_t row1 = row0 + rows_per < B ? row0 + rows_per : B;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l15 = lane & 15, lh = lane >> 4;
  const uint32_t in = static_cast<uint32_t>(nb1) * Q;
  const uint32_t Bu = static_cast<uint32_t>(B);

  // A = Rᵀ[s x k] from the transposed copy: lane holds R[r][k = 32ks + 8lh + e][s = 16w + l15]
  bf16x8 a[4];
  const uint16_t* Rtr = W1t + static_cast<int64_t>(r) * Q * Q;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) a[ks] = frag_ld(Rtr + (16 * w + l15) * Q + 32 * ks + 8 * lh);
  f32x4 accr[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) accr[nt] = zero4();

  // dZ piece: kg = tid>>5, row = tid&31; X piece: row = tid>>4, seg = tid&15
  const int kg = tid >> 5, zrow = tid & 31;
  const uint32_t zcol = (r * 16 + kg) * Bu * 8;
  const int xrow = tid >> 4, seg = tid & 15;
  const uint32_t xcol = r * Q + seg * 8;

  auto gload = [&](u32x4& pz, u32x4& px, int64_t b0) {
    const int64_t bc = b0 < row1 ? b0 : row1 - 1, lim = row1 - bc;
    pz = ldg16(dZ + bc * 8 + clamp_row(zrow, lim) * 8 + zcol);
    px = zero_unless(b0 + xrow < row1, ldg16(X + bc * in + clamp_row(xrow, lim) * in + xcol));
  };
  auto body = [&](u32x4& pz, u32x4& px, int64_t b0) {
    *reinterpret_cast<u32x4*>(&dzs[zrow * XLD + kg * 8]) = pz;
#pragma unroll
    for (int e = 0; e < 8; ++e) dzt[(kg * 8 + e) * TLD + zrow] = half_of(pz, e);
#pragma unroll
    for (int e = 0; e < 8; ++e) xt[(seg * 8 + e) * TLD + xrow] = half_of(px, e);
    __syncthreads();
    gload(pz, px, b0 + 2 * T);
    // dXᵀ[s x b] = Rᵀ[s x k] · dZᵀ[k x b]
    f32x4 accx[2] = {zero4(), zero4()};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        accx[nt] = mfma(a[ks], frag_ld(&dzs[(16 * nt + l15) * XLD + 32 * ks + 8 * lh]), accx[nt]);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      u32x2 v;
      v[0] = pack_bf16x2(accx[nt][0], accx[nt][1]);
      v[1] = pack_bf16x2(accx[nt][2], accx[nt][3]);
      *reinterpret_cast<u32x2*>(&dxs[(16 * nt + l15) * XLD + 16 * w + 4 * lh]) = v;
    }
    // dR[k x s] += dZᵀ[k x b] · X[b x s]
    const bf16x8 A = frag_ld(&dzt[(16 * w + l15) * TLD + 8 * lh]);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
      accr[nt] = mfma(A, frag_ld(&xt[(16 * nt + l15) * TLD + 8 * lh]), accr[nt]);
    __syncthreads();
    const int64_t bc = b0 < row1 ? b0 : row1 - 1, lim = row1 - bc;
    stg16(dX + bc * in + clamp_row(xrow, lim) * in + xcol,
          *reinterpret_cast<const u32x4*>(&dxs[xrow * XLD + seg * 8]));
  };

  if (row0 < row1) {
    const int64_t npairs = (row1 - row0 + 2 * T - 1) / (2 * T);
    u32x4 za, xa, zb, xb;
    gload(za, xa, row0);
    gload(zb, xb, row0 + T);
    drain_prologue();
    for (int64_t k = 0; k < npairs; ++k) {
      body(za, xa, row0 + 2 * k * T);
      body(zb, xb, row0 + (2 * k + 1) * T);
    }
  }
  float* P = partial + (static_cast<int64_t>(chunk) * nb1 + r) * Q * Q;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
#pragma unroll
    for (int v = 0; v < 4; ++v) P[(16 * w + 4 * lh + v) * Q + 16 * nt + l15] = accr[nt][v];
}

// --------------------------------------------------------------------------
// Wt[blk][c][r] = W[blk][r][c] for 128x128 blocks (both factors in one
// launch: blocks [0, nb1) of w1 then [0, nb2) of w2). 32x32 sub-tiles
// through LDS; 256 threads.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void sq_transpose_blocks_kernel(
    const uint16_t* __restrict__ W1, const uint16_t* __restrict__ W2, uint16_t* __restrict__ W1t,
    uint16_t* __restrict__ W2t, int nb1) {
  __shared__ uint16_t tile[32][33];
  const int blk = blockIdx.x >> 4, sub = blockIdx.x & 15;
  const bool first = blk < nb1;
  const int64_t bofs = static_cast<int64_t>(first ? blk : blk - nb1) * Q * Q;
  const uint16_t* src = (first ? W1 : W2) + bofs;
  uint16_t* dst = (first ? W1t : W2t) + bofs;
  const int r0 = (sub >> 2) * 32, c0 = (sub & 3) * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) tile[ty + 8 * i][tx] = src[(r0 + ty + 8 * i) * Q + c0 + tx];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[(c0 + ty + 8 * i) * Q + r0 + tx] = tile[tx][ty + 8 * i];
}

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t clamp64(int64_t v, int64_t lo, int64_t hi) { return v < lo ? lo : (v > hi ? hi : v); }

}  // namespace

bool sq_applicable(int64_t in, int64_t out, int64_t nb1, int64_t nb2, int64_t batch,
                   int dtype_bf16) {
  if (!dtype_bf16) return false;
  if (nb1 != nb2 || nb2 % 8 != 0) return false;
  if (in != nb1 * Q || out != nb2 * Q) return false;
  // 32-bit element offsets inside the kernels
  return batch * out < (int64_t(1) << 31);
}

SqPlan sq_plan(int64_t batch, int64_t nb) {
  SqPlan p;
  const int64_t groups = nb / 8;
  // stage-1 forward: ~2048 workgroups of single blocks
  p.fwd1_chunks = clamp64(2048 / nb, 1, cdiv(batch, 32));
  p.fwd1_rows = round_up(cdiv(batch, p.fwd1_chunks), 32);
  p.fwd1_chunks = cdiv(batch, p.fwd1_rows);
  // stage-2 kernels: one 1024-thread workgroup per CU (256 CUs)
  p.s2_ranges = clamp64(256 / groups, 1, cdiv(batch, 16));
  p.s2_rows = round_up(cdiv(batch, p.s2_ranges), 16);
  p.s2_ranges = cdiv(batch, p.s2_rows);
  // stage-2 weight gradient: groups x 4 p slices x chunks ~ 256 workgroups
  p.w2_chunks = clamp64(256 / (groups * 4), 1, cdiv(batch, 32));
  p.w2_rows = round_up(cdiv(batch, p.w2_chunks), 32);
  p.w2_chunks = cdiv(batch, p.w2_rows);
  // stage-1 backward: 2 workgroups of 8 waves per CU
  p.b1_chunks = clamp64(512 / nb, 1, cdiv(batch, 32));
  p.b1_rows = round_up(cdiv(batch, p.b1_chunks), 32);
  p.b1_chunks = cdiv(batch, p.b1_rows);
  return p;
}

hipError_t sq_launch_transpose_weights(const void* w1, const void* w2, void* w1t, void* w2t,
                                      int64_t nb, hipStream_t s) {
  hipLaunchKernelGGL(sq_transpose_blocks_kernel, dim3(static_cast<unsigned>(2 * nb * 16)), dim3(256),
                     0, s, static_cast<const uint16_t*>(w1), static_cast<const uint16_t*>(w2),
                     static_cast<uint16_t*>(w1t), static_cast<uint16_t*>(w2t), static_cast<int>(nb));
  return hipGetLastError();
}

hipError_t sq_launch_stage1_fwd(const void* x, const void* w1, void* z, int64_t batch, int64_t nb,
                                const SqPlan& p, hipStream_t s) {
  hipLaunchKernelGGL(sq_stage1_fwd_kernel, dim3(static_cast<unsigned>(nb * p.fwd1_chunks)),
                     dim3(256), 0, s, static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(w1), static_cast<uint16_t*>(z), batch,
                     static_cast<int>(nb), p.fwd1_rows);
  return hipGetLastError();
}

hipError_t sq_launch_stage2_fwd(const void* z, const void* w2, void* y, int64_t batch, int64_t nb,
                                int relu, const SqPlan& p, hipStream_t s) {
  hipLaunchKernelGGL(sq_stage2_fwd_kernel, dim3(static_cast<unsigned>(nb / 8 * p.s2_ranges)),
                     dim3(512), 0, s, static_cast<const uint16_t*>(z),
                     static_cast<const uint16_t*>(w2), static_cast<uint16_t*>(y), batch,
                     static_cast<int>(nb), p.s2_rows, relu);
  return hipGetLastError();
}

hipError_t sq_launch_stage2_bwd_data(const void* dy, const void* ymask, const void* w2, void* dz,
                                     int64_t batch, int64_t nb, const SqPlan& p, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(nb / 8 * p.s2_ranges));
  if (ymask)
    hipLaunchKernelGGL(sq_stage2_bwd_data_kernel<true>, grid, dim3(512), 0, s,
                       static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(ymask),
                       static_cast<const uint16_t*>(w2), static_cast<uint16_t*>(dz), batch,
                       static_cast<int>(nb), p.s2_rows);
  else
    hipLaunchKernelGGL(sq_stage2_bwd_data_kernel<false>, grid, dim3(512), 0, s,
                       static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(ymask),
                       static_cast<const uint16_t*>(w2), static_cast<uint16_t*>(dz), batch,
                       static_cast<int>(nb), p.s2_rows);
  return hipGetLastError();
}

hipError_t sq_launch_stage2_bwd_weight(const void* dy, const void* ymask, const void* z,
                                       float* partial, int64_t batch, int64_t nb, const SqPlan& p,
                                       hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(nb / 8 * 4 * p.w2_chunks));
  if (ymask)
    hipLaunchKernelGGL(sq_stage2_bwd_weight_kernel<true>, grid, dim3(512), 0, s,
                       static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(ymask),
                       static_cast<const uint16_t*>(z), partial, batch, static_cast<int>(nb),
                       p.w2_rows);
  else
    hipLaunchKernelGGL(sq_stage2_bwd_weight_kernel<false>, grid, dim3(512), 0, s,
                       static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(ymask),
                       static_cast<const uint16_t*>(z), partial, batch, static_cast<int>(nb),
                       p.w2_rows);
  return hipGetLastError();
}

hipError_t sq_launch_stage1_bwd(const void* dz, const void* x, const void* w1, void* dx,
                                float* partial, int64_t batch, int64_t nb, const SqPlan& p,
                                hipStream_t s) {
  hipLaunchKernelGGL(sq_stage1_bwd_kernel, dim3(static_cast<unsigned>(nb * p.b1_chunks)), dim3(512),
                     0, s, static_cast<const uint16_t*>(dz), static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(w1), static_cast<uint16_t*>(dx), partial, batch,
                     static_cast<int>(nb), p.b1_rows);
  return hipGetLastError();
}

}  // namespace monarch
