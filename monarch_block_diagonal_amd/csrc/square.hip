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
// MFMA fragment from 8 elements at stride `stride` (packed pairwise into
// 32-bit words as they arrive)
__device__ __forceinline__ bf16x8 frag_gather(const uint16_t* p, int64_t stride) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v[i] = static_cast<uint32_t>(p[(2 * i) * stride]) |
           (static_cast<uint32_t>(p[(2 * i + 1) * stride]) << 16);
  bf16x8 r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
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
  __shared__ __attribute__((aligned(16))) uint16_t xs[32 * XLD];
  const int r = blockIdx.x % nb1;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x / nb1) * rows_per;
  const int64_t row1 = row0 + rows_per < B ? row0 + rows_per : B;
  if (row0 >= row1) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l15 = lane & 15, lh = lane >> 4;
  const int64_t in = static_cast<int64_t>(nb1) * Q;

  bf16x8 a[2][4];
  const uint16_t* Rr = W1 + static_cast<int64_t>(r) * Q * Q;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      a[mt][ks] = frag_ld(Rr + (32 * w + 16 * mt + l15) * Q + 32 * ks + 8 * lh);

  u32x4 pre[2];
  auto gload = [&](int64_t b0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int piece = tid + 256 * i, row = piece >> 4, seg = piece & 15;
      const int64_t b = b0 + row;
      pre[i] = b < row1 ? ldg16(X + b * in + r * Q + seg * 8) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int piece = tid + 256 * i, row = piece >> 4, seg = piece & 15;
      *reinterpret_cast<u32x4*>(&xs[row * XLD + seg * 8]) = pre[i];
    }
  };

  gload(row0);
  lstore();
  __syncthreads();
  for (int64_t b0 = row0; b0 < row1; b0 += 32) {
    const bool more = b0 + 32 < row1;
    if (more) gload(b0 + 32);
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
    // feature k = 32w + 16mt + 4lh + v of block r -> panel r*16 + 4w + 2mt + lh/2
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int64_t b = b0 + 16 * nt + l15;
        if (b < row1) {
          const int64_t panel = static_cast<int64_t>(r) * 16 + 4 * w + 2 * mt + (lh >> 1);
          u32x2 v;
          v[0] = pack_bf16x2(acc[mt][nt][0], acc[mt][nt][1]);
          v[1] = pack_bf16x2(acc[mt][nt][2], acc[mt][nt][3]);
          *reinterpret_cast<u32x2*>(Z + (panel * B + b) * 8 + 4 * (lh & 1)) = v;
        }
      }
    __syncthreads();
    if (more) {
      lstore();
      __syncthreads();
    }
  }
}

// --------------------------------------------------------------------------
// stage 2 forward: Y[b, p*b2 + g] = act(sum_t L[g,p,t] Z[b, t*b2 + g])
// --------------------------------------------------------------------------
// 16 waves, 8 L blocks g0..g0+7 per workgroup; wave w: block g0 + w/2, output
// half p in [64*(w&1), +64). Tile: 16 rows. Z panels -> LDS [g][row][t];
// C = Vᵀ[p x b] = L[p x t] · Wᵀ[t x b]; results -> LDS [row][p][g] -> Y in
// 16-byte runs.
__global__ __launch_bounds__(1024) void sq_stage2_fwd_kernel(const uint16_t* __restrict__ Z,
                                                             const uint16_t* __restrict__ W2,
                                                             uint16_t* __restrict__ Y, int64_t B,
                                                             int nb2, int64_t rows_per, int relu) {
  __shared__ __attribute__((aligned(16))) uint16_t ws[8 * 16 * XLD];
  __shared__ __attribute__((aligned(16))) uint16_t ys[16 * YLD];
  const int n_groups = nb2 >> 3;
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int gg = logical % n_groups;
  const int64_t row0 = static_cast<int64_t>(logical / n_groups) * rows_per;
  const int64_t row1 = row0 + rows_per < B ? row0 + rows_per : B;
  if (row0 >= row1) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l15 = lane & 15, lh = lane >> 4;
  const int gl = w >> 1, ph = w & 1;
  const int g = gg * 8 + gl;
  const int64_t out = static_cast<int64_t>(nb2) * Q;
  const int64_t pstride = nb2 >> 3;  // panels between t and t+1

  bf16x8 a[4][4];
  const uint16_t* Lg = W2 + static_cast<int64_t>(g) * Q * Q;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      a[mt][ks] = frag_ld(Lg + (64 * ph + 16 * mt + l15) * Q + 32 * ks + 8 * lh);

  u32x4 pre[2];
  auto gload = [&](int64_t b0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int piece = tid + 1024 * i, t = piece >> 4, row = piece & 15;
      const int64_t b = b0 + row;
      pre[i] = b < row1 ? ldg16(Z + ((t * pstride + gg) * B + b) * 8) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto lscatter = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int piece = tid + 1024 * i, t = piece >> 4, row = piece & 15;
#pragma unroll
      for (int e = 0; e < 8; ++e) ws[(e * 16 + row) * XLD + t] = half_of(pre[i], e);
    }
  };

  gload(row0);
  lscatter();
  __syncthreads();
  for (int64_t b0 = row0; b0 < row1; b0 += 16) {
    const bool more = b0 + 16 < row1;
    if (more) gload(b0 + 16);
    f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 bop = frag_ld(&ws[(gl * 16 + l15) * XLD + 32 * ks + 8 * lh]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma(a[mt][ks], bop, acc[mt]);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float val = acc[mt][v];
        if (relu) val = val > 0.f ? val : 0.f;
        ys[l15 * YLD + (64 * ph + 16 * mt + 4 * lh + v) * 8 + gl] = f32_to_bf16(val);
      }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int piece = tid + 1024 * i, row = piece >> 7, p = piece & 127;
      const int64_t b = b0 + row;
      if (b < row1)
        stg16(Y + b * out + static_cast<int64_t>(p) * nb2 + gg * 8,
              *reinterpret_cast<const u32x4*>(&ys[row * YLD + p * 8]));
    }
    if (more) lscatter();
    __syncthreads();
  }
}

// --------------------------------------------------------------------------
// stage 2 backward, data: dZ[b, t*b2 + g] = sum_p dYe[b, p*b2 + g] L[g,p,t]
// --------------------------------------------------------------------------
// Same tiling as the forward; wave w: block g0 + w/2, t half (w&1).
// dY (masked) -> LDS [g][row][p]; C = dZᵀ[t x b] = Lᵀ[t x p] · dVᵀ[p x b];
// results -> LDS [t][row][g] -> dZ panels (256 B per t).
template <bool MASK>
__global__ __launch_bounds__(1024) void sq_stage2_bwd_data_kernel(
    const uint16_t* __restrict__ dY, const uint16_t* __restrict__ Ym,
    const uint16_t* __restrict__ W2, uint16_t* __restrict__ dZ, int64_t B, int nb2,
    int64_t rows_per) {
  __shared__ __attribute__((aligned(16))) uint16_t dvs[8 * 16 * XLD];
  __shared__ __attribute__((aligned(16))) uint16_t zs[Q * XLD];
  const int n_groups = nb2 >> 3;
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int gg = logical % n_groups;
  const int64_t row0 = static_cast<int64_t>(logical / n_groups) * rows_per;
  const int64_t row1 = row0 + rows_per < B ? row0 + rows_per : B;
  if (row0 >= row1) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l15 = lane & 15, lh = lane >> 4;
  const int gl = w >> 1, th = w & 1;
  const int g = gg * 8 + gl;
  const int64_t out = static_cast<int64_t>(nb2) * Q;
  const int64_t pstride = nb2 >> 3;

  // A = Lᵀ[t x p]: lane holds L[g][p = 32ks + 8lh + e][t = 64th + 16mt + l15]
  bf16x8 a[4][4];
  const uint16_t* Lg = W2 + static_cast<int64_t>(g) * Q * Q;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      a[mt][ks] = frag_gather(Lg + (32 * ks + 8 * lh) * Q + 64 * th + 16 * mt + l15, Q);

  u32x4 pre[2];
  auto gload = [&](int64_t b0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int piece = tid + 1024 * i, row = piece >> 7, p = piece & 127;
      const int64_t b = b0 + row;
      u32x4 v{0u, 0u, 0u, 0u};
      if (b < row1) {
        const int64_t off = b * out + static_cast<int64_t>(p) * nb2 + gg * 8;
        v = ldg16(dY + off);
        if constexpr (MASK) v = apply_mask(v, ldg16(Ym + off));
      }
      pre[i] = v;
    }
  };
  auto lscatter = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int piece = tid + 1024 * i, row = piece >> 7, p = piece & 127;
#pragma unroll
      for (int e = 0; e < 8; ++e) dvs[(e * 16 + row) * XLD + p] = half_of(pre[i], e);
    }
  };

  gload(row0);
  lscatter();
  __syncthreads();
  for (int64_t b0 = row0; b0 < row1; b0 += 16) {
    const bool more = b0 + 16 < row1;
    if (more) gload(b0 + 16);
    f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 bop = frag_ld(&dvs[(gl * 16 + l15) * XLD + 32 * ks + 8 * lh]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma(a[mt][ks], bop, acc[mt]);
    }
    // zs[t][row][g]: 128 u16 per t, pitch XLD
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        zs[(64 * th + 16 * mt + 4 * lh + v) * XLD + l15 * 8 + gl] = f32_to_bf16(acc[mt][v]);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int piece = tid + 1024 * i, t = piece >> 4, row = piece & 15;
      const int64_t b = b0 + row;
      if (b < row1)
        stg16(dZ + ((t * pstride + gg) * B + b) * 8,
              *reinterpret_cast<const u32x4*>(&zs[t * XLD + row * 8]));
    }
    if (more) lscatter();
    __syncthreads();
  }
}

// --------------------------------------------------------------------------
// stage 2 backward, weights: dL[g,p,t] = sum_b dYe[b, p*b2+g] Z[b, t*b2+g]
// --------------------------------------------------------------------------
// Workgroup: 8 L blocks x a 32-wide slice of p x a batch chunk. 16 waves;
// wave w: block g0 + w/2, t half (w&1); accumulators dL[32 p x 64 t] in
// VGPRs. Tile: 32 rows = one K step. dY slice -> LDS [g][p][row], Z panels ->
// LDS [g][t][row] (row-contiguous operands for K = batch). The chunk's sum is
// written as an fp32 partial.
template <bool MASK>
__global__ __launch_bounds__(1024) void sq_stage2_bwd_weight_kernel(
    const uint16_t* __restrict__ dY, const uint16_t* __restrict__ Ym,
    const uint16_t* __restrict__ Z, float* __restrict__ partial, int64_t B, int nb2,
    int64_t rows_per) {
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
  const int gl = w >> 1, th = w & 1;
  const int g = gg * 8 + gl;
  const int64_t out = static_cast<int64_t>(nb2) * Q;
  const int64_t pstride = nb2 >> 3;

  f32x4 acc[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = zero4();

  u32x4 pd, pz[4];
  auto gload = [&](int64_t b0) {
    {
      const int row = tid >> 5, pl = tid & 31;
      const int64_t b = b0 + row;
      u32x4 v{0u, 0u, 0u, 0u};
      if (b < row1) {
        const int64_t off = b * out + static_cast<int64_t>(32 * ps + pl) * nb2 + gg * 8;
        v = ldg16(dY + off);
        if constexpr (MASK) v = apply_mask(v, ldg16(Ym + off));
      }
      pd = v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int piece = tid + 1024 * i, t = piece >> 5, row = piece & 31;
      const int64_t b = b0 + row;
      pz[i] = b < row1 ? ldg16(Z + ((t * pstride + gg) * B + b) * 8) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto lscatter = [&]() {
    {
      const int row = tid >> 5, pl = tid & 31;
#pragma unroll
      for (int e = 0; e < 8; ++e) dvs[(e * 32 + pl) * TLD + row] = half_of(pd, e);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int piece = tid + 1024 * i, t = piece >> 5, row = piece & 31;
#pragma unroll
      for (int e = 0; e < 8; ++e) zst[(e * Q + t) * TLD + row] = half_of(pz[i], e);
    }
  };

  if (row0 < row1) {
    gload(row0);
    lscatter();
  }
  __syncthreads();
  for (int64_t b0 = row0; b0 < row1; b0 += 32) {
    const bool more = b0 + 32 < row1;
    if (more) gload(b0 + 32);
    bf16x8 A[2], Bv[4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) A[mt] = frag_ld(&dvs[(gl * 32 + 16 * mt + l15) * TLD + 8 * lh]);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      Bv[nt] = frag_ld(&zst[(gl * Q + 64 * th + 16 * nt + l15) * TLD + 8 * lh]);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma(A[mt], Bv[nt], acc[mt][nt]);
    __syncthreads();
    if (more) {
      lscatter();
      __syncthreads();
    }
  }
  // partial[chunk][g][p][t]
  float* P = partial + (static_cast<int64_t>(chunk) * nb2 + g) * Q * Q;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        P[(32 * ps + 16 * mt + 4 * lh + v) * Q + 64 * th + 16 * nt + l15] = acc[mt][nt][v];
}

// --------------------------------------------------------------------------
// stage 1 backward: dX_r = dZ_r · R_r and dR_r = sum_b dZ_rᵀ X_r
// --------------------------------------------------------------------------
// One R block and a batch chunk per workgroup, 4 waves; wave w owns dX
// features s in [32w, +32) and dR rows k in [32w, +32). Tile: 32 rows.
// dZ panels -> LDS [row][k] and [k][row]; X -> LDS [s][row].
__global__ __launch_bounds__(256) void sq_stage1_bwd_kernel(
    const uint16_t* __restrict__ dZ, const uint16_t* __restrict__ X,
    const uint16_t* __restrict__ W1, uint16_t* __restrict__ dX, float* __restrict__ partial,
    int64_t B, int nb1, int64_t rows_per) {
  __shared__ __attribute__((aligned(16))) uint16_t dzs[32 * XLD];
  __shared__ __attribute__((aligned(16))) uint16_t dzt[Q * TLD];
  __shared__ __attribute__((aligned(16))) uint16_t xt[Q * TLD];
  __shared__ __attribute__((aligned(16))) uint16_t dxs[32 * XLD];
  const int r = blockIdx.x % nb1;
  const int chunk = blockIdx.x / nb1;
  const int64_t row0 = static_cast<int64_t>(chunk) * rows_per;
  const int64_t row1 = row0 + rows_per < B ? row0 + rows_per : B;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l15 = lane & 15, lh = lane >> 4;
  const int64_t in = static_cast<int64_t>(nb1) * Q;

  // A = Rᵀ[s x k]: lane holds R[r][k = 32ks + 8lh + e][s = 32w + 16mt + l15]
  bf16x8 a[2][4];
  const uint16_t* Rr = W1 + static_cast<int64_t>(r) * Q * Q;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      a[mt][ks] = frag_gather(Rr + (32 * ks + 8 * lh) * Q + 32 * w + 16 * mt + l15, Q);
  f32x4 accr[2][8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) accr[mt][nt] = zero4();

  u32x4 pz[2], px[2];
  auto gload = [&](int64_t b0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int piece = tid + 256 * i;
      {
        const int kg = piece >> 5, row = piece & 31;
        const int64_t b = b0 + row;
        pz[i] = b < row1 ? ldg16(dZ + ((static_cast<int64_t>(r) * 16 + kg) * B + b) * 8)
                         : u32x4{0u, 0u, 0u, 0u};
      }
      {
        const int row = piece >> 4, seg = piece & 15;
        const int64_t b = b0 + row;
        px[i] = b < row1 ? ldg16(X + b * in + r * Q + seg * 8) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int piece = tid + 256 * i;
      {
        const int kg = piece >> 5, row = piece & 31;
        *reinterpret_cast<u32x4*>(&dzs[row * XLD + kg * 8]) = pz[i];
#pragma unroll
        for (int e = 0; e < 8; ++e) dzt[(kg * 8 + e) * TLD + row] = half_of(pz[i], e);
      }
      {
        const int row = piece >> 4, seg = piece & 15;
#pragma unroll
        for (int e = 0; e < 8; ++e) xt[(seg * 8 + e) * TLD + row] = half_of(px[i], e);
      }
    }
  };

  if (row0 < row1) {
    gload(row0);
    lstore();
  }
  __syncthreads();
  for (int64_t b0 = row0; b0 < row1; b0 += 32) {
    const bool more = b0 + 32 < row1;
    if (more) gload(b0 + 32);
    // dXᵀ[s x b] = Rᵀ[s x k] · dZᵀ[k x b]
    f32x4 accx[2][2] = {{zero4(), zero4()}, {zero4(), zero4()}};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 bop[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        bop[nt] = frag_ld(&dzs[(16 * nt + l15) * XLD + 32 * ks + 8 * lh]);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) accx[mt][nt] = mfma(a[mt][ks], bop[nt], accx[mt][nt]);
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        u32x2 v;
        v[0] = pack_bf16x2(accx[mt][nt][0], accx[mt][nt][1]);
        v[1] = pack_bf16x2(accx[mt][nt][2], accx[mt][nt][3]);
        *reinterpret_cast<u32x2*>(&dxs[(16 * nt + l15) * XLD + 32 * w + 16 * mt + 4 * lh]) = v;
      }
    // dR[k x s] += dZᵀ[k x b] · X[b x s]
    {
      bf16x8 A[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) A[mt] = frag_ld(&dzt[(32 * w + 16 * mt + l15) * TLD + 8 * lh]);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const bf16x8 Bv = frag_ld(&xt[(16 * nt + l15) * TLD + 8 * lh]);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) accr[mt][nt] = mfma(A[mt], Bv, accr[mt][nt]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int piece = tid + 256 * i, row = piece >> 4, seg = piece & 15;
      const int64_t b = b0 + row;
      if (b < row1)
        stg16(dX + b * in + r * Q + seg * 8, *reinterpret_cast<const u32x4*>(&dxs[row * XLD + seg * 8]));
    }
    if (more) lstore();
    __syncthreads();
  }
  float* P = partial + (static_cast<int64_t>(chunk) * nb1 + r) * Q * Q;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        P[(32 * w + 16 * mt + 4 * lh + v) * Q + 16 * nt + l15] = accr[mt][nt][v];
}

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t clamp64(int64_t v, int64_t lo, int64_t hi) { return v < lo ? lo : (v > hi ? hi : v); }

}  // namespace

bool sq_applicable(int64_t in, int64_t out, int64_t nb1, int64_t nb2, int dtype_bf16) {
  if (!dtype_bf16) return false;
  if (nb1 != nb2 || nb2 % 8 != 0) return false;
  return in == nb1 * Q && out == nb2 * Q;
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
  // stage-1 backward: 2 workgroups per CU (2 waves per SIMD)
  p.b1_chunks = clamp64(512 / nb, 1, cdiv(batch, 32));
  p.b1_rows = round_up(cdiv(batch, p.b1_chunks), 32);
  p.b1_chunks = cdiv(batch, p.b1_rows);
  return p;
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
                     dim3(1024), 0, s, static_cast<const uint16_t*>(z),
                     static_cast<const uint16_t*>(w2), static_cast<uint16_t*>(y), batch,
                     static_cast<int>(nb), p.s2_rows, relu);
  return hipGetLastError();
}

hipError_t sq_launch_stage2_bwd_data(const void* dy, const void* ymask, const void* w2, void* dz,
                                     int64_t batch, int64_t nb, const SqPlan& p, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(nb / 8 * p.s2_ranges));
  if (ymask)
    hipLaunchKernelGGL(sq_stage2_bwd_data_kernel<true>, grid, dim3(1024), 0, s,
                       static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(ymask),
                       static_cast<const uint16_t*>(w2), static_cast<uint16_t*>(dz), batch,
                       static_cast<int>(nb), p.s2_rows);
  else
    hipLaunchKernelGGL(sq_stage2_bwd_data_kernel<false>, grid, dim3(1024), 0, s,
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
    hipLaunchKernelGGL(sq_stage2_bwd_weight_kernel<true>, grid, dim3(1024), 0, s,
                       static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(ymask),
                       static_cast<const uint16_t*>(z), partial, batch, static_cast<int>(nb),
                       p.w2_rows);
  else
    hipLaunchKernelGGL(sq_stage2_bwd_weight_kernel<false>, grid, dim3(1024), 0, s,
                       static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(ymask),
                       static_cast<const uint16_t*>(z), partial, batch, static_cast<int>(nb),
                       p.w2_rows);
  return hipGetLastError();
}

hipError_t sq_launch_stage1_bwd(const void* dz, const void* x, const void* w1, void* dx,
                                float* partial, int64_t batch, int64_t nb, const SqPlan& p,
                                hipStream_t s) {
  hipLaunchKernelGGL(sq_stage1_bwd_kernel, dim3(static_cast<unsigned>(nb * p.b1_chunks)), dim3(256),
                     0, s, static_cast<const uint16_t*>(dz), static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(w1), static_cast<uint16_t*>(dx), partial, batch,
                     static_cast<int>(nb), p.b1_rows);
  return hipGetLastError();
}

}  // namespace monarch
