// Fast path for bf16 Monarch layers whose four block dimensions are all 128
// (in = mid = out = 128*b, nblocks1 = nblocks2 = b, b in {32, 64, 128}): the
// square Definition C.3 family (scatterbrain issues page, "Definition C.3"
// thread) at block size 128, e.g. n = 16384 with 128 blocks.
//
// At this block size every stage is HBM-bound (64 flop per byte moved at the
// I/O width against a bf16 MFMA ridge near 300), so the kernels are built
// around data movement:
//
//  * Tile-major panel layout for the intermediates: the batch is cut into
//    16-row tiles, and a tile stores each 8-feature panel as one run of its
//    rows: feature f of row b sits at (b - b%16)*F + ((f/8)*rt + b%16)*8 +
//    f%8 (F features per row, rt = 16 rows, fewer in a last partial tile).
//    A 16-byte piece holds 8 features of one row, one panel of a tile is a
//    256-byte run, and the runs a kernel reads together lie within one
//    tile's F*32 bytes whatever the batch: with a panel-major order (stride
//    B*16 bytes between panels) some batch sizes map those runs onto few
//    memory channels and cache sets. The saved stage-2
//    input (z) is W = P·Z in this layout, W[b, g*128 + t] = Z[b, t*b2 + g]:
//    the stride permutation of the "hypercube" thread is applied once, by the
//    stage-1 kernel's stores, and every stage-2 kernel reads whole pieces of
//    one L block. The gradient of stage 2's output (dV, from dY) uses the
//    same layout; dZ, read by the stage-1 backward, is in Z order.
//  * The caller's row-major Y / dY hold the L blocks of one (row, p) side by
//    side, so the stage-2 forward owns 32 blocks to write 64-byte runs, and a
//    transpose pass moves dY into dV panels with 256-byte runs. Narrower runs
//    cost up to 2-3x in achieved bandwidth on this memory system. Workgroups
//    that share cache lines are mapped onto one XCD (workgroups are
//    dispatched round-robin over the 8 XCDs).
//  * Weights stay in VGPRs for the whole launch (persistent workgroups over
//    a row range); MFMA v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
//    Where a lane's MFMA operand is one 16-byte piece of a panel or a row it
//    is loaded straight from global memory into registers.
//  * Weight gradients accumulate in registers over a batch chunk per
//    workgroup; chunks are summed afterwards in a fixed order.
#include <type_traits>

#include "common.h"
#include "square.h"

namespace monarch {
namespace {

constexpr int Q = 128;        // block size
constexpr int XLD = Q + 8;    // LDS pitch (elements) of [row][feature] tiles
constexpr int TLD = 32 + 8;   // LDS pitch of [feature][32 rows] tiles

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// streaming load for the last reader of a tensor in the pass
__device__ __forceinline__ u32x4 ldg16_nt(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void stg16(uint16_t* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
// streaming store for final outputs that no later kernel of the pass reads
__device__ __forceinline__ void stg16_nt(uint16_t* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ bf16x8 frag_ld(const uint16_t* p) {
  return as_bf16x8(*reinterpret_cast<const u16x8*>(p));
}
// 8 elements at a stride of one 128-element block row: a fragment of a
// transposed weight block, gathered once when a workgroup starts
__device__ __forceinline__ bf16x8 frag_gather(const uint16_t* p) {
  u16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = p[e * 128];
  return as_bf16x8(v);
}
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

// Empty asm statements that claim to modify a value: code placed after one
// cannot be scheduled before the load that produced the value. Used to wait
// once for everything a prologue issued (weights and the first prefetched
// tiles): the wait counts the compiler inserts at a loop head are the minimum
// over its predecessors, so without it the prologue's issue order would set
// them and drain the prefetch slots on every iteration. Also placed before a
// select on a prefetched value, which would otherwise be hoisted up to the
// load and wait for the prefetch right after issuing it.
template <typename T> __device__ __forceinline__ void pin(T& v) { asm volatile("" : "+v"(v)); }
template <typename T, int N> __device__ __forceinline__ void pin(T (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) pin(v[i]);
}

__device__ __forceinline__ int clamp_row(int row, int64_t lim) {
  return row < lim ? row : static_cast<int>(lim - 1);
}
__device__ __forceinline__ u32x4 zero_unless(bool keep, u32x4 v) {
  return keep ? v : u32x4{0u, 0u, 0u, 0u};
}

// Row b of the tile-major panel layout (F features per row, B rows): piece
// (b, panel P) is at base + P*rt8 elements.
struct PanelRow {
  uint32_t base;   // tile start * F + (b % 16) * 8
  uint32_t rt8;    // 8 * rows of b's tile
};
__device__ __forceinline__ PanelRow panel_row(int64_t b, uint32_t F, uint32_t Bu) {
  const uint32_t bu = static_cast<uint32_t>(b), t0 = bu & ~15u;
  const uint32_t rt = Bu - t0 < 16u ? Bu - t0 : 16u;
  return PanelRow{t0 * F + (bu & 15u) * 8u, rt * 8u};
}

// --------------------------------------------------------------------------
// stage 1 forward, stored in stage 2's input order:
//   W[b, g*128 + t] = Z[b, t*b2 + g],  Z[b, r*128 + k] = sum_s R[r,k,s] X[b, r*128 + s]
// --------------------------------------------------------------------------
// Workgroup: 8 R blocks r0..r0+7 x a row range; wave w owns block r0 + w
// (R fragments: 128 VGPRs). Tile: 16 rows; the MFMA B operands (X[b][8 s])
// are 16-byte pieces of X rows, loaded straight into registers two tiles
// ahead. C = Zᵀ[k x b] = R[k x s] · Xᵀ[s x b]. Output (r, k) is W-feature
// (g, t) = ((r*128 + k) % b2, (r*128 + k) / b2); the 8 blocks cover 1024/b2
// consecutive t of every g, i.e. 128 whole 8-t pieces per row, staged in LDS
// [piece][row][t%8] and stored in 256-byte runs.
template <int LNB>
__global__ __launch_bounds__(512) void sq_stage1_fwd_kernel(const uint16_t* __restrict__ X,
                                                            const uint16_t* __restrict__ W1,
                                                            uint16_t* __restrict__ Wz, int64_t B,
                                                            int64_t rows_per) {
  constexpr int NB = 1 << LNB;
  constexpr int NPC = Q / NB;         // 8-t pieces per g covered by one workgroup
  constexpr int T = 16;
  constexpr int ZP = T * 8 + 8;       // LDS pitch of one staged piece
  constexpr uint32_t in = NB * Q;
  __shared__ __attribute__((aligned(16))) uint16_t zs[Q * ZP];
  constexpr int n_rg = NB / 8;
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int rg = logical % n_rg;
  const int64_t row0 = static_cast<int64_t>(logical / n_rg) * rows_per;
  const int64_t row1 = row0 + rows_per < B ? row0 + rows_per : B;
  if (row0 >= row1) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l15 = lane & 15, lh = lane >> 4;
  const int r = rg * 8 + w;
  const uint32_t Bu = static_cast<uint32_t>(B);

  // A = R_r[k x s]: lane holds R[r][k = 16mt + l15][s = 32ks + 8lh ..]
  bf16x8 a[8][4];
  const uint16_t* Rr = W1 + static_cast<int64_t>(r) * Q * Q;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a[mt][ks] = frag_ld(Rr + (16 * mt + l15) * Q + 32 * ks + 8 * lh);

  const uint32_t xcol = r * Q + 8 * lh;
  // staged pieces: pid = (tid>>4) + 32i, row = tid&15 -> panel (pid/NPC)*16 + rg*NPC + pid%NPC
  const int spid = tid >> 4, srow = tid & 15;

  auto gload = [&](u32x4(&pre)[4], int64_t b0) {
    const int64_t bc = b0 < row1 ? b0 : row1 - 1, lim = row1 - bc;
    const uint16_t* base = X + (bc + clamp_row(l15, lim)) * in + xcol;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) pre[ks] = ldg16(base + 32 * ks);
  };
  auto body = [&](u32x4(&cur)[4], int64_t b0) {
    pin(cur);
    f32x4 acc[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[mt] = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 bop;
      __builtin_memcpy(&bop, &cur[ks], sizeof(bop));
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) acc[mt] = mfma(a[mt][ks], bop, acc[mt]);
    }
    gload(cur, b0 + 2 * T);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int v = 0; v < 4; v += 2) {
        const uint32_t pk = pack_bf16x2(acc[mt][v], acc[mt][v + 1]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int k = 16 * mt + 4 * lh + v + h;
          const int g = k & (NB - 1);
          const int tl = w * NPC + (k >> LNB);       // t relative to the workgroup's first t
          zs[(g * NPC + (tl >> 3)) * ZP + l15 * 8 + (tl & 7)] =
              static_cast<uint16_t>(h ? pk >> 16 : pk & 0xffffu);
        }
      }
    __syncthreads();
    const int64_t bc = b0 < row1 ? b0 : row1 - 1, lim = row1 - bc;
    const PanelRow pr = panel_row(bc + clamp_row(srow, lim), in, Bu);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pid = spid + 32 * i;
      const uint32_t panel = (pid / NPC) * 16 + rg * NPC + pid % NPC;
      stg16_nt(Wz + pr.base + panel * pr.rt8,
               *reinterpret_cast<const u32x4*>(&zs[pid * ZP + srow * 8]));
    }
    __syncthreads();
  };

  const int64_t npairs = (row1 - row0 + 2 * T - 1) / (2 * T);
  u32x4 pa[4], pb[4];
  gload(pa, row0);
  gload(pb, row0 + T);
  pin(a);
  pin(pa);
  pin(pb);
  for (int64_t k = 0; k < npairs; ++k) {
    body(pa, row0 + 2 * k * T);
    body(pb, row0 + (2 * k + 1) * T);
  }
}

// --------------------------------------------------------------------------
// stage 2 forward: Y[b, p*b2 + g] = act(sum_t L[g,p,t] W[b, g*128 + t])
// --------------------------------------------------------------------------
// Workgroup: 32 L blocks g0..g0+31 x a 32-wide slice of p x a row range, so
// each (row, p) of Y gets a 64-byte run. 8 waves; wave w owns blocks
// g0+4w..+3 for the 32 p of the slice (L fragments: 128 VGPRs). Row tile: 16
// rows; the t contraction runs in 4 chunks of 32, in an order rotated by the
// p slice. The MFMA B operands (W[b][8 t] of one block) are 16-byte pieces
// of the W panels, loaded straight into registers two chunks ahead.
// C = Vᵀ[p x b] = L[p x t] · Wᵀ[t x b]; after 4 chunks the tile -> LDS
// [row][p][g] -> Y.
constexpr int Y2LD = 32 * 32 + 8;    // pitch of [row][32 p][32 g]

__global__ __launch_bounds__(512) void sq_stage2_fwd_kernel(const uint16_t* __restrict__ Wz,
                                                            const uint16_t* __restrict__ W2,
                                                            uint16_t* __restrict__ Y, int64_t B,
                                                            int nb2, int64_t rows_per, int relu) {
  constexpr int T = 16;
  __shared__ __attribute__((aligned(16))) uint16_t ys[T * Y2LD];
  const int n_gq = nb2 >> 5;
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int ps = logical & 3;
  const int gq = (logical >> 2) % n_gq;
  const int64_t row0 = static_cast<int64_t>((logical >> 2) / n_gq) * rows_per;
  const int64_t row1 = row0 + rows_per < B ? row0 + rows_per : B;
  if (row0 >= row1) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l15 = lane & 15, lh = lane >> 4;
  const uint32_t out = static_cast<uint32_t>(nb2) * Q;
  const uint32_t Bu = static_cast<uint32_t>(B);

  // The four workgroups of a block group (one per p slice) read the same W
  // pieces. Each takes the tile's t chunks in its own rotated order (chunk j
  // of the tile is t chunk (j + ps) % 4), so they do not request the same
  // lines at the same moment; the lines are L2 hits for the later ones.
  // a[g][mt][j] = L[g0+4w+g][p = 32ps + 16mt + l15][t = 32((j + ps) % 4) + 8lh ..]
  bf16x8 a[4][2][4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint16_t* Lg = W2 + static_cast<int64_t>(gq * 32 + 4 * w + g) * Q * Q;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        a[g][mt][j] = frag_ld(Lg + (32 * ps + 16 * mt + l15) * Q + 32 * ((j + ps) & 3) + 8 * lh);
  }

  // operand pieces: panel (g0+4w+g)*16 + 4tc + lh, row b0 + l15
  const uint32_t wpanel = (gq * 32 + 4 * w) * 16 + lh;
  // Y pieces: id = tid + 512i: q4 = id&3, pl = (id>>2)&31, row = id>>7 (+4i)
  const int yq4 = tid & 3, ypl = (tid >> 2) & 31, yrow = tid >> 7;
  const uint32_t ycol = (32 * ps + ypl) * nb2 + gq * 32 + yq4 * 8;

  // chunk c of the row range: tile c>>2, t chunk (c + ps) & 3
  auto gload = [&](u32x4(&pre)[4], int64_t c) {
    const int64_t b0 = row0 + (c >> 2) * T;
    const int64_t bc = b0 < row1 ? b0 : row1 - 1, lim = row1 - bc;
    const PanelRow pr = panel_row(bc + clamp_row(l15, lim), out, Bu);
    const uint16_t* base = Wz + pr.base + (wpanel + 4 * static_cast<uint32_t>((c + ps) & 3)) * pr.rt8;
#pragma unroll
    for (int g = 0; g < 4; ++g) pre[g] = ldg16(base + g * 16 * pr.rt8);   // next block: +16 panels
  };

  f32x4 acc[4][2];
  const int64_t ntiles = (row1 - row0 + T - 1) / T;
  const int64_t nchunks = ntiles * 4;
  u32x4 pa[4], pb[4];
  gload(pa, 0);
  gload(pb, 1);
  pin(a);
  pin(pa);
  pin(pb);
  auto step = [&](auto tcc, u32x4(&cur)[4], int64_t tile) {
    constexpr int tc = decltype(tcc)::value;
    const int64_t c = tile * 4 + tc;
    pin(cur);
    if constexpr (tc == 0) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) acc[g][mt] = zero4();
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x8 bop;
      __builtin_memcpy(&bop, &cur[g], sizeof(bop));
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) acc[g][mt] = mfma(a[g][mt][tc], bop, acc[g][mt]);
    }
    gload(cur, c + 2 < nchunks ? c + 2 : nchunks - 1);
    if constexpr (tc == 3) {
      // tile done: results -> ys[row][p][g], then Y
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int v = 0; v < 4; v += 2) {
            float v0 = acc[g][mt][v], v1 = acc[g][mt][v + 1];
            if (relu) {
              v0 = v0 > 0.f ? v0 : 0.f;
              v1 = v1 > 0.f ? v1 : 0.f;
            }
            const uint32_t pk = pack_bf16x2(v0, v1);
            const int pl = 16 * mt + 4 * lh + v;
            ys[l15 * Y2LD + pl * 32 + 4 * w + g] = static_cast<uint16_t>(pk & 0xffffu);
            ys[l15 * Y2LD + (pl + 1) * 32 + 4 * w + g] = static_cast<uint16_t>(pk >> 16);
          }
      __syncthreads();
      const int64_t b0 = row0 + tile * T;
      const int64_t bc = b0 < row1 ? b0 : row1 - 1, lim = row1 - bc;
      uint16_t* yb = Y + bc * out + ycol;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        stg16_nt(yb + clamp_row(yrow + 4 * i, lim) * out,
                 *reinterpret_cast<const u32x4*>(&ys[(yrow + 4 * i) * Y2LD + ypl * 32 + yq4 * 8]));
      __syncthreads();
    }
  };
  for (int64_t tile = 0; tile < ntiles; ++tile) {
    step(std::integral_constant<int, 0>{}, pa, tile);
    step(std::integral_constant<int, 1>{}, pb, tile);
    step(std::integral_constant<int, 2>{}, pa, tile);
    step(std::integral_constant<int, 3>{}, pb, tile);
  }
}

// --------------------------------------------------------------------------
// dV panels: dV[b, g*128 + p] = dYe[b, p*b2 + g]  (block-major gradient of
// stage 2's output; dYe = dY masked by Y > 0 after a fused ReLU)
// --------------------------------------------------------------------------
// The inverse stride permutation scatters one L block's outputs with stride
// b2 through each row of Y, so a kernel owning a few blocks would read dY in
// short runs. This pass reads dY rows in 256-byte runs (all blocks of 16 p at
// once), transposes 8x8 bf16 blocks in registers and writes dV (feature
// i = g*128 + p) in the panel layout through LDS in 256-byte runs. Both
// backward stage-2 kernels then read dV contiguously.
// Tile: RT = 256/GO rows x 16 p x 8*GO blocks (GO = min(16, b2/8) block
// octets); 512 threads, one 8x8 block each; one tile per workgroup. The
// staging row is XOR-swizzled with the block octet, so the 16-byte stores of
// lanes with consecutive octets land on distinct banks.
__global__ __launch_bounds__(512) void sq_dv_panels_kernel(const uint16_t* __restrict__ dY,
                                                           const uint16_t* __restrict__ Ym,
                                                           uint16_t* __restrict__ dV, int64_t B,
                                                           int nb2) {
  __shared__ __attribute__((aligned(16))) u32x4 st[4096];   // [g][po][row] 16-byte pieces
  const int GO = nb2 >= 128 ? 16 : nb2 >> 3;
  const int RT = 256 / GO;
  const int n_gt = nb2 / (8 * GO);            // block groups per row
  int bid = blockIdx.x;
  const int gt = bid % n_gt;
  bid /= n_gt;
  const int pt = bid & 7;                     // 16-p tile
  const int64_t b0 = static_cast<int64_t>(bid >> 3) * RT;
  const int tid = threadIdx.x;
  const int go = tid % GO, po = (tid / GO) & 1, row = tid / (2 * GO);
  const uint32_t out = static_cast<uint32_t>(nb2) * Q;
  const int64_t b = b0 + row < B ? b0 + row : B - 1;
  const int64_t src = b * out + static_cast<int64_t>(16 * pt + 8 * po) * nb2 + (gt * GO + go) * 8;
  u32x4 in[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) in[i] = ldg16_nt(dY + src + i * nb2);
  if (Ym) {
#pragma unroll
    for (int i = 0; i < 8; ++i) in[i] = relu_mask_bf16(in[i], ldg16_nt(Ym + src + i * nb2));
  }
  u32x2 lo[8], hi[8];
  transpose4x8(*reinterpret_cast<const u32x4(*)[4]>(&in[0]), lo);
  transpose4x8(*reinterpret_cast<const u32x4(*)[4]>(&in[4]), hi);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    st[((go * 8 + e) * 2 + po) * RT + (row ^ go)] = u32x4{lo[e][0], lo[e][1], hi[e][0], hi[e][1]};
  __syncthreads();
  const int n_pieces = 8 * GO * 2 * RT;   // 4096
  for (int id = tid; id < n_pieces; id += 512) {
    const int r = id % RT, q = (id / RT) & 1, gl = id / (2 * RT);
    const int64_t bb = b0 + r;
    if (bb < B) {
      const uint32_t panel = static_cast<uint32_t>(gt * GO * 8 + gl) * 16 + 2 * pt + q;
      const PanelRow pr = panel_row(bb, out, static_cast<uint32_t>(B));
      stg16(dV + pr.base + panel * pr.rt8, st[(gl * 2 + q) * RT + (r ^ (gl >> 3))]);
    }
  }
}

// --------------------------------------------------------------------------
// stage 2 backward, data: dZ[b, t*b2 + g] = sum_p dV[b, g*128 + p] L[g,p,t]
// --------------------------------------------------------------------------
// 8 waves, 8 L blocks g0..g0+7 per workgroup; wave w owns block g0 + w (all
// t; Lᵀ fragments gathered from L at the start: 128 VGPRs). Tile: 16 rows; the
// MFMA B operands (dV_g[b][8 p]) are 16-byte pieces of the dV panels, loaded
// straight into registers two tiles ahead. C = dZᵀ[t x b] = Lᵀ[t x p] ·
// dVᵀ[p x b]; results -> LDS [t][row][g] -> dZ panels (256-byte runs).
__global__ __launch_bounds__(512) void sq_stage2_bwd_data_kernel(
    const uint16_t* __restrict__ dV, const uint16_t* __restrict__ W2,
    uint16_t* __restrict__ dZ, int64_t B, int nb2, int64_t rows_per) {
  constexpr int T = 16;
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
  const uint32_t Bu = static_cast<uint32_t>(B);
  const uint32_t pstride = nb2 >> 3;

  // A = Lᵀ[t x p]: lane holds L[g][p = 32ks + 8lh + e][t = 16mt + l15]
  bf16x8 a[8][4];
  const uint16_t* Lg = W2 + static_cast<int64_t>(g) * Q * Q;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a[mt][ks] = frag_gather(Lg + (32 * ks + 8 * lh) * Q + 16 * mt + l15);

  const uint32_t F = static_cast<uint32_t>(nb2) * Q;
  // operand pieces: panel g*16 + 4ks + lh, row b0 + l15
  const uint32_t vpanel = g * 16 + lh;
  // dZ pieces: t = (tid>>4) + 32i, row = tid&15; panel (t*b2 + g0)/8
  const int zt = tid >> 4, zrow = tid & 15;
  const uint32_t zpanel = zt * pstride + gg;
  const uint32_t zstep = 32 * pstride;   // panels

  auto gload = [&](u32x4(&pre)[4], int64_t b0) {
    const int64_t bc = b0 < row1 ? b0 : row1 - 1, lim = row1 - bc;
    const PanelRow pr = panel_row(bc + clamp_row(l15, lim), F, Bu);
    const uint16_t* base = dV + pr.base + vpanel * pr.rt8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) pre[ks] = ldg16_nt(base + 4 * ks * pr.rt8);   // +4 panels
  };
  auto body = [&](u32x4(&cur)[4], int64_t b0) {
    pin(cur);
    f32x4 acc[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[mt] = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 bop;
      __builtin_memcpy(&bop, &cur[ks], sizeof(bop));
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) acc[mt] = mfma(a[mt][ks], bop, acc[mt]);
    }
    gload(cur, b0 + 2 * T);
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
    const PanelRow pr = panel_row(bc + clamp_row(zrow, lim), F, Bu);
    uint16_t* zb = dZ + pr.base + zpanel * pr.rt8;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      stg16_nt(zb + i * zstep * pr.rt8,
               *reinterpret_cast<const u32x4*>(&zs[(zt + 32 * i) * XLD + zrow * 8]));
    __syncthreads();
  };

  const int64_t npairs = (row1 - row0 + 2 * T - 1) / (2 * T);
  u32x4 pa[4], pb[4];
  gload(pa, row0);
  gload(pb, row0 + T);
  pin(a);
  pin(pa);
  pin(pb);
  for (int64_t k = 0; k < npairs; ++k) {
    body(pa, row0 + 2 * k * T);
    body(pb, row0 + (2 * k + 1) * T);
  }
}

// --------------------------------------------------------------------------
// stage 2 backward, weights: dL[g,p,t] = sum_b dV[b, g*128 + p] W[b, g*128 + t]
// --------------------------------------------------------------------------
// Workgroup: one L block x a batch chunk, all p and t. 4 waves; wave w owns
// p in [32w, +32): accumulators dL[32 p x 128 t] in VGPRs. Tile: 32 rows =
// one K step; two tiles in flight in registers. dV and W are both
// block-major panels: waves 0-1 load dV, waves 2-3 load W, each thread 4
// rows of one panel. Both MFMA operands need consecutive batch rows per
// lane, so a 4x8 register transpose gives 8-byte LDS writes of
// [feature][position] tiles. A sum over rows may take them in any order:
// position 4rq + i holds row rq + 8i in both operands, so every load
// instruction reads whole 128-byte lines (8 consecutive rows of a panel).
// The chunk's sum is written as an fp32 partial.
__device__ __forceinline__ int fl_row(int f) { return f * TLD + (f >> 3) * 8; }  // LDS row of feature f

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void sq_stage2_bwd_weight_kernel(
    const uint16_t* __restrict__ dV, const uint16_t* __restrict__ Wz, float* __restrict__ partial,
    int64_t B, int nb2, int64_t rows_per) {
  constexpr int T = 32;
  constexpr int TS = Q * TLD + Q;   // one operand's [128][positions] tile (+ skew)
  __shared__ __attribute__((aligned(16))) uint16_t ts[2 * TS];
  const int g = blockIdx.x % nb2;
  const int chunk = blockIdx.x / nb2;
  const int64_t row0 = static_cast<int64_t>(chunk) * rows_per;
  const int64_t row1 = row0 + rows_per < B ? row0 + rows_per : B;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l15 = lane & 15, lh = lane >> 4;

  f32x4 acc[2][8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = zero4();

  // loader role: thread (rq = lt&7, pl = lt>>3) loads rows rq + 8i of panel
  // g*16 + pl (features 8pl ..) of dV or W
  const bool is_w = w >= 2;
  const int lt = tid & 127, rq = lt & 7, pl = lt >> 3;
  const uint16_t* src = is_w ? Wz : dV;
  const uint32_t panel = g * 16 + pl;
  const uint32_t F = static_cast<uint32_t>(nb2) * Q, Bu = static_cast<uint32_t>(B);
  uint16_t* tdst = &ts[(is_w ? TS : 0) + fl_row(pl * 8) + 4 * rq];

  auto gload = [&](u32x4(&pre)[4], int64_t b0) {
    const int64_t bc = b0 < row1 ? b0 : row1 - 1, lim = row1 - bc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const PanelRow pr = panel_row(bc + clamp_row(rq + 8 * i, lim), F, Bu);
      pre[i] = ldg16_nt(src + pr.base + panel * pr.rt8);
    }
  };
  auto body = [&](u32x4(&pre)[4], int64_t b0) {
    pin(pre);
    // dV rows past the range were loaded clamped: zero them (W rows stay)
#pragma unroll
    for (int i = 0; i < 4; ++i) pre[i] = zero_unless(is_w || b0 + rq + 8 * i < row1, pre[i]);
    u32x2 tr[8];
    transpose4x8(pre, tr);
#pragma unroll
    for (int e = 0; e < 8; ++e) *reinterpret_cast<u32x2*>(tdst + e * TLD) = tr[e];
    __syncthreads();
    gload(pre, b0 + 2 * T);
    bf16x8 A[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) A[mt] = frag_ld(&ts[fl_row(32 * w + 16 * mt + l15) + 8 * lh]);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const bf16x8 Bv = frag_ld(&ts[TS + fl_row(16 * nt + l15) + 8 * lh]);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) acc[mt][nt] = mfma(A[mt], Bv, acc[mt][nt]);
    }
    __syncthreads();
  };

  if (row0 < row1) {
    const int64_t npairs = (row1 - row0 + 2 * T - 1) / (2 * T);
    u32x4 pa[4], pb[4];
    gload(pa, row0);
    gload(pb, row0 + T);
    pin(pa);
    pin(pb);
    for (int64_t k = 0; k < npairs; ++k) {
      body(pa, row0 + 2 * k * T);
      body(pb, row0 + (2 * k + 1) * T);
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
        P[(32 * w + 16 * mt + 4 * lh + v) * Q + 16 * nt + l15] = acc[mt][nt][v];
}

// --------------------------------------------------------------------------
// stage 1 backward: dX_r = dZ_r · R_r and dR_r = sum_b dZ_rᵀ X_r
// --------------------------------------------------------------------------
// One R block and a batch chunk per workgroup, 8 waves; wave w owns dX
// features s in [16w, +16) and dR rows k in [16w, +16). Tile: 64 rows; two
// tiles in flight in registers. Waves 0-3 load dZ, waves 4-7 load X: each
// thread 4 rows (rq + 16i) of one 8-feature piece, so a load instruction
// reads 256-byte runs, and a 4x8 register transpose gives 8-byte LDS writes
// for the row-contiguous copies the dR product needs (K = batch). A sum
// over rows may take them in any order: position 4rq + i holds row rq + 16i
// in both dR operands. dZ also goes to LDS row-major (dX operand); X rows
// past the range are zeroed, so dR only sums real rows.
constexpr int T1 = 64;            // stage-1 backward row tile
constexpr int PLD = T1 + 8;       // LDS pitch of [feature][64 positions] tiles

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void sq_stage1_bwd_kernel(
    const uint16_t* __restrict__ dZ, const uint16_t* __restrict__ X,
    const uint16_t* __restrict__ W1, uint16_t* __restrict__ dX, float* __restrict__ partial,
    int64_t B, int nb1, int64_t rows_per) {
  constexpr int T = T1;
  __shared__ __attribute__((aligned(16))) uint16_t dzs[T * XLD];   // [row][k]
  __shared__ __attribute__((aligned(16))) uint16_t dxs[T * XLD];   // [row][s]
  __shared__ __attribute__((aligned(16))) uint16_t ts[2][Q * PLD];  // dZ: [k][pos], X: [s][pos]
  const int r = blockIdx.x % nb1;
  const int chunk = blockIdx.x / nb1;
  const int64_t row0 = static_cast<int64_t>(chunk) * rows_per;
  const int64_t row1 = row0 + rows_per < B ? row0 + rows_per : B;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l15 = lane & 15, lh = lane >> 4;
  const uint32_t in = static_cast<uint32_t>(nb1) * Q;

  // A = Rᵀ[s x k], gathered from R: lane holds R[r][k = 32ks + 8lh + e][s = 16w + l15]
  bf16x8 a[4];
  const uint16_t* Rr = W1 + static_cast<int64_t>(r) * Q * Q;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) a[ks] = frag_gather(Rr + (32 * ks + 8 * lh) * Q + 16 * w + l15);
  f32x4 accr[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) accr[nt] = zero4();

  // loader role: dZ (panel r*16 + oct, 16-byte row stride) or X (columns
  // r*128 + 8*oct, row stride in); rows rq + 16i of the tile
  const bool is_x = w >= 4;
  const int lt = tid & 255;
  const int rq = is_x ? lt >> 4 : lt & 15;
  const int oct = is_x ? lt & 15 : lt >> 4;
  const uint16_t* src = is_x ? X + r * Q + oct * 8 : dZ;
  const uint32_t zpanel = r * 16 + oct, Bu = static_cast<uint32_t>(B);
  uint16_t* tdst = &ts[is_x ? 1 : 0][(oct * 8) * PLD + 4 * rq];
  // dX store pieces: seg = tid&15, rows (tid>>4) + 32i
  const int xseg = tid & 15, xrow = tid >> 4;

  auto gload = [&](u32x4(&pre)[4], int64_t b0) {
    const int64_t bc = b0 < row1 ? b0 : row1 - 1, lim = row1 - bc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = bc + clamp_row(rq + 16 * i, lim);
      const PanelRow pr = panel_row(row, in, Bu);
      const uint32_t off = is_x ? static_cast<uint32_t>(row) * in : pr.base + zpanel * pr.rt8;
      pre[i] = ldg16_nt(src + off);
    }
  };
  auto body = [&](u32x4(&pre)[4], int64_t b0) {
    pin(pre);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pre[i] = zero_unless(!is_x || b0 + rq + 16 * i < row1, pre[i]);
    if (!is_x) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4*>(&dzs[(rq + 16 * i) * XLD + oct * 8]) = pre[i];
    }
    u32x2 tr[8];
    transpose4x8(pre, tr);
#pragma unroll
    for (int e = 0; e < 8; ++e) *reinterpret_cast<u32x2*>(tdst + e * PLD) = tr[e];
    __syncthreads();
    gload(pre, b0 + 2 * T);
    // dXᵀ[s x b] = Rᵀ[s x k] · dZᵀ[k x b], 4 column tiles of 16 rows
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      f32x4 accx = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        accx = mfma(a[ks], frag_ld(&dzs[(16 * nt + l15) * XLD + 32 * ks + 8 * lh]), accx);
      u32x2 v;
      v[0] = pack_bf16x2(accx[0], accx[1]);
      v[1] = pack_bf16x2(accx[2], accx[3]);
      *reinterpret_cast<u32x2*>(&dxs[(16 * nt + l15) * XLD + 16 * w + 4 * lh]) = v;
    }
    // dR[k x s] += dZᵀ[k x pos] · X[pos x s]
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 A = frag_ld(&ts[0][(16 * w + l15) * PLD + 32 * kk + 8 * lh]);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
        accr[nt] = mfma(A, frag_ld(&ts[1][(16 * nt + l15) * PLD + 32 * kk + 8 * lh]), accr[nt]);
    }
    __syncthreads();
    const int64_t bc = b0 < row1 ? b0 : row1 - 1, lim = row1 - bc;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      stg16_nt(dX + bc * in + clamp_row(xrow + 32 * i, lim) * in + r * Q + xseg * 8,
               *reinterpret_cast<const u32x4*>(&dxs[(xrow + 32 * i) * XLD + xseg * 8]));
  };

  if (row0 < row1) {
    const int64_t npairs = (row1 - row0 + 2 * T - 1) / (2 * T);
    u32x4 pa[4], pb[4];
    gload(pa, row0);
    gload(pb, row0 + T);
    pin(a);
    pin(pa);
    pin(pb);
    for (int64_t k = 0; k < npairs; ++k) {
      body(pa, row0 + 2 * k * T);
      body(pb, row0 + (2 * k + 1) * T);
    }
  }
  float* P = partial + (static_cast<int64_t>(chunk) * nb1 + r) * Q * Q;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
#pragma unroll
    for (int v = 0; v < 4; ++v) P[(16 * w + 4 * lh + v) * Q + 16 * nt + l15] = accr[nt][v];
}

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t clamp64(int64_t v, int64_t lo, int64_t hi) { return v < lo ? lo : (v > hi ? hi : v); }

}  // namespace

bool sq_applicable(int64_t in, int64_t out, int64_t nb1, int64_t nb2, int64_t batch,
                   int dtype_bf16) {
  if (!dtype_bf16) return false;
  // the stage-1 forward writes whole 8-t pieces from 8 R blocks: 128/nb must
  // be a whole number, and the stage-2 forward takes blocks 32 at a time
  if (nb1 != nb2 || (nb2 != 32 && nb2 != 64 && nb2 != 128)) return false;
  if (in != nb1 * Q || out != nb2 * Q) return false;
  // 32-bit element offsets inside the kernels
  return batch * out < (int64_t(1) << 31);
}

SqPlan sq_plan(int64_t batch, int64_t nb) {
  SqPlan p;
  const int64_t groups = nb / 32;   // 32-block groups of the stage-2 kernels
  // stage-1 forward: nb/8 block groups x row ranges ~ one workgroup per CU
  p.fwd1_chunks = clamp64(256 / (nb / 8), 1, cdiv(batch, 16));
  p.fwd1_rows = round_up(cdiv(batch, p.fwd1_chunks), 16);
  p.fwd1_chunks = cdiv(batch, p.fwd1_rows);
  // stage-2 data kernels: groups x 4 slices x row ranges ~ one workgroup per CU
  p.s2_ranges = clamp64(256 / (groups * 4), 1, cdiv(batch, 16));
  p.s2_rows = round_up(cdiv(batch, p.s2_ranges), 16);
  p.s2_ranges = cdiv(batch, p.s2_rows);
  // stage-2 backward data: nb/8 block groups x row ranges ~ one workgroup per CU
  p.d2_ranges = clamp64(256 / (nb / 8), 1, cdiv(batch, 16));
  p.d2_rows = round_up(cdiv(batch, p.d2_ranges), 16);
  p.d2_ranges = cdiv(batch, p.d2_rows);
  // stage-2 weight gradient: nb blocks x chunks ~ three 4-wave workgroups per CU
  p.w2_chunks = clamp64(768 / nb, 1, cdiv(batch, 32));
  p.w2_rows = round_up(cdiv(batch, p.w2_chunks), 32);
  p.w2_chunks = cdiv(batch, p.w2_rows);
  // stage-1 backward: 2 workgroups of 8 waves per CU
  p.b1_chunks = clamp64(512 / nb, 1, cdiv(batch, T1));
  p.b1_rows = round_up(cdiv(batch, p.b1_chunks), T1);
  p.b1_chunks = cdiv(batch, p.b1_rows);
  return p;
}

hipError_t sq_launch_stage1_fwd(const void* x, const void* w1, void* z, int64_t batch, int64_t nb,
                                const SqPlan& p, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(nb / 8 * p.fwd1_chunks)), block(512);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint16_t* wp = static_cast<const uint16_t*>(w1);
  uint16_t* zp = static_cast<uint16_t*>(z);
  switch (nb) {
    case 32: hipLaunchKernelGGL(sq_stage1_fwd_kernel<5>, grid, block, 0, s, xp, wp, zp, batch, p.fwd1_rows); break;
    case 64: hipLaunchKernelGGL(sq_stage1_fwd_kernel<6>, grid, block, 0, s, xp, wp, zp, batch, p.fwd1_rows); break;
    case 128: hipLaunchKernelGGL(sq_stage1_fwd_kernel<7>, grid, block, 0, s, xp, wp, zp, batch, p.fwd1_rows); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t sq_launch_stage2_fwd(const void* z, const void* w2, void* y, int64_t batch, int64_t nb,
                                int relu, const SqPlan& p, hipStream_t s) {
  hipLaunchKernelGGL(sq_stage2_fwd_kernel, dim3(static_cast<unsigned>(nb / 32 * 4 * p.s2_ranges)),
                     dim3(512), 0, s, static_cast<const uint16_t*>(z),
                     static_cast<const uint16_t*>(w2), static_cast<uint16_t*>(y), batch,
                     static_cast<int>(nb), p.s2_rows, relu);
  return hipGetLastError();
}

hipError_t sq_launch_dv_panels(const void* dy, const void* ymask, void* dv, int64_t batch,
                               int64_t nb, hipStream_t s) {
  const int64_t GO = nb >= 128 ? 16 : nb / 8;
  const int64_t RT = 256 / GO;
  const int64_t grid = cdiv(batch, RT) * 8 * (nb / (8 * GO));
  hipLaunchKernelGGL(sq_dv_panels_kernel, dim3(static_cast<unsigned>(grid)), dim3(512), 0, s,
                     static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(ymask),
                     static_cast<uint16_t*>(dv), batch, static_cast<int>(nb));
  return hipGetLastError();
}

hipError_t sq_launch_stage2_bwd_data(const void* dv, const void* w2, void* dz, int64_t batch,
                                     int64_t nb, const SqPlan& p, hipStream_t s) {
  hipLaunchKernelGGL(sq_stage2_bwd_data_kernel, dim3(static_cast<unsigned>(nb / 8 * p.d2_ranges)),
                     dim3(512), 0, s, static_cast<const uint16_t*>(dv),
                     static_cast<const uint16_t*>(w2), static_cast<uint16_t*>(dz), batch,
                     static_cast<int>(nb), p.d2_rows);
  return hipGetLastError();
}

hipError_t sq_launch_stage2_bwd_weight(const void* dv, const void* z, float* partial,
                                       int64_t batch, int64_t nb, const SqPlan& p, hipStream_t s) {
  hipLaunchKernelGGL(sq_stage2_bwd_weight_kernel,
                     dim3(static_cast<unsigned>(nb * p.w2_chunks)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(dv), static_cast<const uint16_t*>(z), partial,
                     batch, static_cast<int>(nb), p.w2_rows);
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
