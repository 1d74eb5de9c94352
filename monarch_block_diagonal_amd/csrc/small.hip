// Fused path for bf16 Monarch layers with 32 x 32 blocks and whole rows of
// at most 1024 features (in = mid = out = 32*b, nblocks1 = nblocks2 = b,
// b in {8, 16, 32}): the square Definition C.3 family (scatterbrain issues
// page, "Definition C.3" thread) at block size 32, e.g. n = 1024 with 32
// blocks.
//
// At this size a row is at most 2 KB, so a workgroup holds a tile of 16 whole
// rows in LDS and runs both stages on it: the stride permutation between the
// stages ("hypercube" thread) and the output permutation become LDS index
// arithmetic, and every HBM access is a 16-byte piece of a row-major tile.
//
//  * Forward (one launch): X -> stage 1 -> W = P·Z in LDS -> stage 2 -> Y. It
//    stores W as the saved z (row-major, W[b, g*32 + t] = Z[b, t*b + g]) and
//    Y; HBM traffic is X read once, z and Y written once.
//  * Backward data (one launch): dY (masked by Y > 0 after a fused ReLU) ->
//    dV[b, g*32 + p] = dY[b, p*b + g] in LDS -> dZ = dV·L per block, stored
//    in Z order -> dX = dZ·R per block. It also stores dV and dZ (row-major).
//  * Weight gradients (one launch for both factors): dL[g] = sum_b
//    dV[b, g-block]ᵀ z[b, g-block] and dR[r] = sum_b dZ[b, r-block]ᵀ
//    X[b, r-block] over batch chunks, one fp32 partial per chunk, summed in a
//    fixed order afterwards.
//
// Each of the 8 waves owns b/8 blocks of each factor; a block's 32 x 32
// weights are two MFMA operands (v_mfma_f32_16x16x32_bf16: K = 32 is one
// block's contraction) held in VGPRs for the whole launch.
#include "common.h"
#include "small.h"

namespace monarch {
namespace {

constexpr int SB = 32;   // block size
constexpr int ST = 16;   // rows per tile

__device__ __forceinline__ u32x4 lds16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ bf16x8 as_op(u32x4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
}
__device__ __forceinline__ bf16x8 ld_op(const uint16_t* p) {
  return as_op(*reinterpret_cast<const u32x4*>(p));
}
// 8 elements at a stride of one block row: a fragment of a transposed block
__device__ __forceinline__ bf16x8 gather_op(const uint16_t* p) {
  u16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = p[e * SB];
  return as_bf16x8(v);
}
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}

// Copies `rows` rows of an LDS tile (pitch LDP) to a row-major global tile,
// 16-byte pieces.
template <int N, int LDP>
__device__ __forceinline__ void store_tile(uint16_t* dst, const uint16_t* src, int rows, int tid) {
  constexpr int PPR = N / 8;   // pieces per row
  for (int i = tid; i < rows * PPR; i += 512) {
    const int r = i / PPR, c = i % PPR;
    *reinterpret_cast<u32x4*>(dst + static_cast<int64_t>(r) * N + c * 8) = lds16(src + r * LDP + c * 8);
  }
}

// --------------------------------------------------------------------------
// forward: Z[b, r*32 + k] = sum_s R[r,k,s] X[b, r*32 + s]
//          W[b, g*32 + t] = Z[b, t*NB + g]                       (saved z)
//          Y[b, p*NB + g] = act(sum_t L[g,p,t] W[b, g*32 + t])
// --------------------------------------------------------------------------
// Wave w owns blocks w*BPW .. +BPW-1 of both factors. Stage 1: C = Zᵀ[k x b]
// = R_r[k x s] · Xᵀ[s x b], the X operand (8 s of one row) loaded straight
// from HBM; results go to the W tile at their permuted positions. Stage 2:
// C = Vᵀ[p x b] = L_g[p x t] · Wᵀ[t x b], operands from the W tile; results
// go to the Y tile at their permuted positions.
template <int NB>
__global__ __launch_bounds__(512) void sm_fwd_kernel(const uint16_t* __restrict__ X,
                                                     const uint16_t* __restrict__ W1,
                                                     const uint16_t* __restrict__ W2,
                                                     uint16_t* __restrict__ Y,
                                                     uint16_t* __restrict__ Z, int64_t B,
                                                     int relu) {
  constexpr int N = NB * SB, BPW = NB / 8, LDP = N + 8;
  __shared__ __attribute__((aligned(16))) uint16_t ws[ST * LDP];
  __shared__ __attribute__((aligned(16))) uint16_t ys[ST * LDP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l15 = lane & 15, lh = lane >> 4;

  // A operands: R[r][k = 16mt + l15][s = 8lh ..], L[g][p = 16mt + l15][t = 8lh ..]
  bf16x8 ra[BPW][2], la[BPW][2];
#pragma unroll
  for (int j = 0; j < BPW; ++j)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int64_t off = (static_cast<int64_t>(w * BPW + j) * SB + 16 * mt + l15) * SB + 8 * lh;
      ra[j][mt] = ld_op(W1 + off);
      la[j][mt] = ld_op(W2 + off);
    }

  const int64_t ntiles = (B + ST - 1) / ST;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t b0 = tile * ST;
    const int rows = B - b0 < ST ? static_cast<int>(B - b0) : ST;
    // rows past the end repeat the last row; they are never stored
    const int64_t brow = b0 + (l15 < rows ? l15 : rows - 1);
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const int r = w * BPW + j;
      const bf16x8 xop = ld_op(X + brow * N + r * SB + 8 * lh);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const f32x4 acc = mfma(ra[j][mt], xop);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int f = r * SB + 16 * mt + 4 * lh + v;   // Z feature
          ws[l15 * LDP + (f % NB) * SB + f / NB] = f32_to_bf16(acc[v]);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const int g = w * BPW + j;
      const bf16x8 wop = ld_op(&ws[l15 * LDP + g * SB + 8 * lh]);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const f32x4 acc = mfma(la[j][mt], wop);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int p = 16 * mt + 4 * lh + v;
          const float y = relu && !(acc[v] > 0.f) ? 0.f : acc[v];
          ys[l15 * LDP + p * NB + g] = f32_to_bf16(y);
        }
      }
    }
    store_tile<N, LDP>(Z + b0 * N, ws, rows, tid);
    __syncthreads();
    store_tile<N, LDP>(Y + b0 * N, ys, rows, tid);
    __syncthreads();
  }
}

// --------------------------------------------------------------------------
// backward, data: dV[b, g*32 + p] = dYe[b, p*NB + g]
//                 dZ[b, t*NB + g] = sum_p dV[b, g*32 + p] L[g,p,t]
//                 dX[b, r*32 + s] = sum_k dZ[b, r*32 + k] R[r,k,s]
// --------------------------------------------------------------------------
// dYe = dY masked by Y > 0 after a fused ReLU. Both products take C[b x .]
// with the activation tile as the A operand (8 consecutive features of one
// row, read from LDS) and a transposed weight block as the B operand
// (gathered once per launch). dV and dZ are also stored row-major for the
// weight gradients; the dV tile's LDS is reused for dX.
template <int NB>
__global__ __launch_bounds__(512) void sm_bwd_data_kernel(
    const uint16_t* __restrict__ dY, const uint16_t* __restrict__ Ym,
    const uint16_t* __restrict__ W1, const uint16_t* __restrict__ W2, uint16_t* __restrict__ dX,
    uint16_t* __restrict__ dV, uint16_t* __restrict__ dZ, int64_t B) {
  constexpr int N = NB * SB, BPW = NB / 8, LDP = N + 8, PPR = N / 8;
  __shared__ __attribute__((aligned(16))) uint16_t vs[ST * LDP];   // dV, then dX
  __shared__ __attribute__((aligned(16))) uint16_t zs[ST * LDP];   // dZ (Z order)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l15 = lane & 15, lh = lane >> 4;

  // B operands: L[g][p = 8lh + e][t = 16nt + l15], R[r][k = 8lh + e][s = 16nt + l15]
  bf16x8 lb[BPW][2], rb[BPW][2];
#pragma unroll
  for (int j = 0; j < BPW; ++j)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int64_t off = static_cast<int64_t>(w * BPW + j) * SB * SB + 8 * lh * SB + 16 * nt + l15;
      lb[j][nt] = gather_op(W2 + off);
      rb[j][nt] = gather_op(W1 + off);
    }

  const int64_t ntiles = (B + ST - 1) / ST;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t b0 = tile * ST;
    const int rows = B - b0 < ST ? static_cast<int>(B - b0) : ST;
    // dY pieces: 8 features p*NB + g0 .. g0+7 of one row (NB >= 8) -> dV
    // positions (g0+e)*32 + p; rows past the end read the last row
    for (int i = tid; i < ST * PPR; i += 512) {
      const int r = i / PPR, c = i % PPR;
      const int64_t src = (b0 + (r < rows ? r : rows - 1)) * N + c * 8;
      u32x4 v = *reinterpret_cast<const u32x4*>(dY + src);
      if (Ym) v = relu_mask_bf16(v, *reinterpret_cast<const u32x4*>(Ym + src));
      const int p = (c * 8) / NB, g0 = (c * 8) % NB;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        vs[r * LDP + (g0 + e) * SB + p] = static_cast<uint16_t>(v[e >> 1] >> (16 * (e & 1)));
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const int g = w * BPW + j;
      const bf16x8 aop = ld_op(&vs[l15 * LDP + g * SB + 8 * lh]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const f32x4 acc = mfma(aop, lb[j][nt]);   // rows 4lh + v, t = 16nt + l15
#pragma unroll
        for (int v = 0; v < 4; ++v)
          zs[(4 * lh + v) * LDP + (16 * nt + l15) * NB + g] = f32_to_bf16(acc[v]);
      }
    }
    store_tile<N, LDP>(dV + b0 * N, vs, rows, tid);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const int r = w * BPW + j;
      const bf16x8 aop = ld_op(&zs[l15 * LDP + r * SB + 8 * lh]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const f32x4 acc = mfma(aop, rb[j][nt]);   // rows 4lh + v, s = 16nt + l15
#pragma unroll
        for (int v = 0; v < 4; ++v)
          vs[(4 * lh + v) * LDP + r * SB + 16 * nt + l15] = f32_to_bf16(acc[v]);
      }
    }
    store_tile<N, LDP>(dZ + b0 * N, zs, rows, tid);
    __syncthreads();
    store_tile<N, LDP>(dX + b0 * N, vs, rows, tid);
    __syncthreads();
  }
}

// --------------------------------------------------------------------------
// weight gradients: partial[c][blk][i][j] = sum over the rows of chunk c of
// A[b, blk*32 + i] Bm[b, blk*32 + j], with (A, Bm) = (dV, z) for dL and
// (dZ, X) for dR
// --------------------------------------------------------------------------
// Workgroup: one factor, two adjacent blocks (so that every row is read as
// one 128-byte run), one chunk of rows; 8 waves, wave w owns the 16 x 16
// output tile ((w / 2) % 2, w % 2) of block w / 4 of the pair. K step: 32
// rows. Threads 0-255 load the A rows and 256-511 the Bm rows (one 16-byte
// piece of 8 features each, the next step's piece in flight) and store them
// transposed, [feature][row], so that both MFMA operands (8 consecutive rows
// of one feature) are 16-byte LDS reads.
template <int NB>
__global__ __launch_bounds__(512) void sm_wgrad_kernel(
    const uint16_t* __restrict__ dV, const uint16_t* __restrict__ Zs,
    const uint16_t* __restrict__ dZ, const uint16_t* __restrict__ X,
    float* __restrict__ part_l, float* __restrict__ part_r, int64_t B, int64_t chunk) {
  static_assert(NB % 2 == 0, "block pairs");
  constexpr int N = NB * SB, KT = 32, TP = KT + 8;
  __shared__ __attribute__((aligned(16))) uint16_t ts[2][2 * SB * TP];
  int bid = blockIdx.x;
  const int blk = (bid % (NB / 2)) * 2;   // first block of the pair
  bid /= NB / 2;
  const int fac = bid & 1;
  const int64_t split = bid >> 1;
  const int64_t r0 = split * chunk;
  const int64_t r1 = r0 + chunk < B ? r0 + chunk : B;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l15 = lane & 15, lh = lane >> 4;
  const int op = tid >> 8, lrow = (tid & 255) >> 3, lcol = (tid & 7) * 8;
  const uint16_t* src = (op ? (fac ? X : Zs) : (fac ? dZ : dV)) + blk * SB + lcol;
  uint16_t* dst = &ts[op][lcol * TP + lrow];
  const int pb = w >> 2, mi = (w >> 1) & 1, ni = w & 1;   // block of the pair, tile

  // rows past the chunk read as zero (they add nothing to the sums)
  auto load = [&](int64_t b0) -> u32x4 {
    const int64_t row = b0 + lrow;
    return row < r1 ? *reinterpret_cast<const u32x4*>(src + row * N) : u32x4{0u, 0u, 0u, 0u};
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  u32x4 cur = load(r0);
  for (int64_t b0 = r0; b0 < r1; b0 += KT) {
    const u32x4 nxt = b0 + KT < r1 ? load(b0 + KT) : cur;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      dst[e * TP] = static_cast<uint16_t>(cur[e >> 1] >> (16 * (e & 1)));
    __syncthreads();
    const bf16x8 a = ld_op(&ts[0][(SB * pb + 16 * mi + l15) * TP + 8 * lh]);
    const bf16x8 b = ld_op(&ts[1][(SB * pb + 16 * ni + l15) * TP + 8 * lh]);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    __syncthreads();
    cur = nxt;
  }
  float* part = (fac ? part_r : part_l) + (split * NB + blk + pb) * SB * SB;
#pragma unroll
  for (int v = 0; v < 4; ++v) part[(16 * mi + 4 * lh + v) * SB + 16 * ni + l15] = acc[v];
}

// about two workgroups per CU (each holds two 16-row tiles of LDS)
int64_t grid_for(int64_t batch) {
  const int64_t tiles = (batch + ST - 1) / ST;
  return tiles < 512 ? tiles : 512;
}

}  // namespace

bool sm_applicable(int64_t in, int64_t out, int64_t nb1, int64_t nb2, int64_t batch,
                   int dtype_bf16) {
  if (!dtype_bf16 || nb1 != nb2) return false;
  if (nb1 != 8 && nb1 != 16 && nb1 != 32) return false;
  if (in != nb1 * SB || out != nb2 * SB) return false;
  return batch > 0 && batch * out < (int64_t(1) << 31);
}

hipError_t sm_launch_fwd(const void* x, const void* w1, const void* w2, void* y, void* z,
                         int64_t batch, int64_t nb, int relu, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(grid_for(batch))), block(512);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint16_t* r = static_cast<const uint16_t*>(w1);
  const uint16_t* l = static_cast<const uint16_t*>(w2);
  uint16_t* yp = static_cast<uint16_t*>(y);
  uint16_t* zp = static_cast<uint16_t*>(z);
  switch (nb) {
    case 8: hipLaunchKernelGGL(sm_fwd_kernel<8>, grid, block, 0, s, xp, r, l, yp, zp, batch, relu); break;
    case 16: hipLaunchKernelGGL(sm_fwd_kernel<16>, grid, block, 0, s, xp, r, l, yp, zp, batch, relu); break;
    case 32: hipLaunchKernelGGL(sm_fwd_kernel<32>, grid, block, 0, s, xp, r, l, yp, zp, batch, relu); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

void sm_wgrad_split(int64_t batch, int64_t* splits, int64_t* chunk) {
  // chunks of at least 256 rows (a multiple of the 32-row step), at most 64
  int64_t c = (batch + 63) / 64;
  if (c < 256) c = 256;
  c = (c + 31) / 32 * 32;
  *chunk = c;
  *splits = (batch + c - 1) / c;
}

hipError_t sm_launch_wgrad(const void* dv, const void* z, const void* dz, const void* x,
                           float* part_l, float* part_r, int64_t batch, int64_t nb,
                           hipStream_t s) {
  int64_t splits, chunk;
  sm_wgrad_split(batch, &splits, &chunk);
  const dim3 grid(static_cast<unsigned>(2 * (nb / 2) * splits)), block(512);
  const uint16_t* a = static_cast<const uint16_t*>(dv);
  const uint16_t* b = static_cast<const uint16_t*>(z);
  const uint16_t* c = static_cast<const uint16_t*>(dz);
  const uint16_t* d = static_cast<const uint16_t*>(x);
  switch (nb) {
    case 8: hipLaunchKernelGGL(sm_wgrad_kernel<8>, grid, block, 0, s, a, b, c, d, part_l, part_r, batch, chunk); break;
    case 16: hipLaunchKernelGGL(sm_wgrad_kernel<16>, grid, block, 0, s, a, b, c, d, part_l, part_r, batch, chunk); break;
    case 32: hipLaunchKernelGGL(sm_wgrad_kernel<32>, grid, block, 0, s, a, b, c, d, part_l, part_r, batch, chunk); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t sm_launch_bwd_data(const void* dy, const void* ymask, const void* w1, const void* w2,
                              void* dx, void* dv, void* dz, int64_t batch, int64_t nb,
                              hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(grid_for(batch))), block(512);
  const uint16_t* dyp = static_cast<const uint16_t*>(dy);
  const uint16_t* m = static_cast<const uint16_t*>(ymask);
  const uint16_t* r = static_cast<const uint16_t*>(w1);
  const uint16_t* l = static_cast<const uint16_t*>(w2);
  uint16_t* dxp = static_cast<uint16_t*>(dx);
  uint16_t* dvp = static_cast<uint16_t*>(dv);
  uint16_t* dzp = static_cast<uint16_t*>(dz);
  switch (nb) {
    case 8: hipLaunchKernelGGL(sm_bwd_data_kernel<8>, grid, block, 0, s, dyp, m, r, l, dxp, dvp, dzp, batch); break;
    case 16: hipLaunchKernelGGL(sm_bwd_data_kernel<16>, grid, block, 0, s, dyp, m, r, l, dxp, dvp, dzp, batch); break;
    case 32: hipLaunchKernelGGL(sm_bwd_data_kernel<32>, grid, block, 0, s, dyp, m, r, l, dxp, dvp, dzp, batch); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace monarch
