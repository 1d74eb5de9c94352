// Tiled strided batched GEMM for the generic Monarch path (gfx950).
//
// Same contract as generic_gemm_kernel (GemmArgs in kernels.h: a batch of
// independent block products at affine offsets, ReLU on the result, fp32
// batch-split partials, the optional column split), for operands whose
// elements are contiguous along one tile dimension:
//   A: K-contiguous (mode 1) or M-contiguous (mode 2),
//   B: K-contiguous (mode 1) or N-contiguous (mode 2).
// Every step of the Monarch product meets this once the saved intermediate
// is kept in stage 2's order and dY is gathered into block-major order (both
// arranged by the planner), so operand tiles move as 16-byte pieces.
//
// Workgroup: 256 threads = 4 waves in a WM x WN grid; each wave owns FM x FN
// 16x16 MFMA tiles (bf16: v_mfma_f32_16x16x32_bf16, fp32:
// v_mfma_f32_16x16x4_f32; fp32 accumulation). K step: 64 (bf16) or 32
// (fp32). Both operand tiles sit in LDS as [row][k] with a 16-byte skew per
// 8 rows. A mode-1 piece is one 16-byte store; a mode-2 thread loads four
// consecutive k rows of one 16-byte piece and transposes them in registers,
// so it also writes 8- or 16-byte [row][k] runs. The next K tile is loaded
// into registers while the current one is multiplied. Consecutive workgroups
// walk the blocks of one output tile first (the stage-2 outputs of the
// blocks interleave in memory) and, when the grid allows, share an XCD.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace monarch {
namespace {

constexpr int TT = 256;

template <typename T>
struct Cfg {
  static constexpr bool kBf16 = std::is_same<T, uint16_t>::value;
  static constexpr int VEC = 16 / static_cast<int>(sizeof(T));  // elements per 16-byte piece
  static constexpr int TK = kBf16 ? 64 : 32;                     // K step
  static constexpr int LD = TK + VEC;                             // LDS row pitch (elements)
  // LDS offset of tile row r: pitch plus a 16-byte skew per 8 rows, which
  // spreads the transposed stores and the fragment reads over the banks
  static __device__ __host__ constexpr int rowoff(int r) { return r * LD + (r >> 3) * VEC; }
};

__device__ __forceinline__ void pin(u32x4& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ u32x4 ld16(const void* p) { return *static_cast<const u32x4*>(p); }

// One operand tile (A: rows = M, B: rows = N) of ROWS x TK elements.
//   mode 1 (K-contiguous): unit = one 16-byte piece (row r, k piece kp);
//   mode 2 (row-contiguous): unit = four k rows of one 16-byte row piece.
// init() resolves each unit's row address once (rows past `lim` are clamped
// to an in-range row and later stored as zeros); `sk` is the K stride.
template <typename T, int MODE, int ROWS>
struct Tile {
  using C = Cfg<T>;
  static constexpr int VEC = C::VEC, TK = C::TK;
  static constexpr int UNITS = MODE == 1 ? ROWS * (TK / VEC) : (ROWS / VEC) * (TK / 4);
  static constexpr int NU = (UNITS + TT - 1) / TT;
  static constexpr int NR = MODE == 1 ? NU : 4 * NU;
  static constexpr int LDS = C::rowoff(ROWS);
  static_assert(MODE == 1 || ROWS % VEC == 0, "row pieces");

  const T* row[NU];   // row address of each unit (k = 0)
  bool rowok[NU];
  int64_t sk, kb, ke;
  u32x4 reg[NR];

  __device__ __forceinline__ static bool active(int q) {
    return UNITS % TT == 0 || static_cast<int>(threadIdx.x) + TT * q < UNITS;
  }
  __device__ __forceinline__ static int unit_row(int q) {
    const int id = threadIdx.x + TT * q;
    return MODE == 1 ? id / (TK / VEC) : (id % (ROWS / VEC)) * VEC;
  }
  __device__ __forceinline__ static int unit_k(int q) {
    const int id = threadIdx.x + TT * q;
    return MODE == 1 ? (id % (TK / VEC)) * VEC : 4 * (id / (ROWS / VEC));
  }

  // row r of the operand sits at base + (r / ns)*hi + (r % ns)*lo (ns > 0)
  // or base + r*lo
  __device__ __forceinline__ void init(const T* base, int64_t r0, int64_t lim, int64_t lo,
                                       int64_t hi, int64_t ns, int64_t sk_, int64_t kb_,
                                       int64_t ke_) {
    sk = sk_, kb = kb_, ke = ke_;
#pragma unroll
    for (int q = 0; q < NU; ++q) {
      const int64_t gr = r0 + unit_row(q);
      rowok[q] = gr < lim;
      const int64_t r = rowok[q] ? gr : 0;
      row[q] = base + (ns > 0 ? (r / ns) * hi + (r % ns) * lo : r * lo);
    }
  }

  __device__ __forceinline__ void load(int64_t k0) {
#pragma unroll
    for (int q = 0; q < NU; ++q) {
      if (!active(q)) continue;
      if constexpr (MODE == 1) {
        int64_t gk = k0 + unit_k(q);
        gk = gk < ke ? gk : kb;
        reg[q] = ld16(row[q] + gk);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int64_t gk = k0 + unit_k(q) + i;
          gk = gk < ke ? gk : kb;
          reg[4 * q + i] = ld16(row[q] + gk * sk);
        }
      }
    }
  }

  // units loaded clamped (row past `lim`, k past `ke`) are stored as zeros
  __device__ __forceinline__ void store(T* s, int64_t k0) {
#pragma unroll
    for (int q = 0; q < NU; ++q) {
      if (!active(q)) continue;
      const int r = unit_row(q), k = unit_k(q);
      if constexpr (MODE == 1) {
        pin(reg[q]);
        const bool keep = rowok[q] && k0 + k < ke;
        const u32x4 v = keep ? reg[q] : u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(s + C::rowoff(r) + k) = v;
      } else {
        u32x4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pin(reg[4 * q + i]);
          const bool keep = rowok[q] && k0 + k + i < ke;
          v[i] = keep ? reg[4 * q + i] : u32x4{0u, 0u, 0u, 0u};
        }
        if constexpr (C::kBf16) {
          u32x2 tr[8];
          transpose4x8(v, tr);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            *reinterpret_cast<u32x2*>(s + C::rowoff(r + e) + k) = tr[e];
        } else {
          u32x4 tr[4];
          transpose4x4(v, tr);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            *reinterpret_cast<u32x4*>(s + C::rowoff(r + e) + k) = tr[e];
        }
      }
    }
  }
};

template <typename T, int AM, int BMD, int WM, int WN, int FM, int FN>
__global__ __launch_bounds__(TT) void tiled_gemm_kernel(GemmArgs p, int64_t m_tiles,
                                                        int64_t n_tiles, int remap) {
  using C = Cfg<T>;
  constexpr int TM = WM * FM * 16, TN = WN * FN * 16, TK = C::TK;
  static_assert(WM * WN == 4, "four waves");
  using TA = Tile<T, AM, TM>;
  using TB = Tile<T, BMD, TN>;
  __shared__ __attribute__((aligned(16))) T As[TA::LDS];
  __shared__ __attribute__((aligned(16))) T Bs[TB::LDS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int l15 = lane & 15, lh = lane >> 4;

  int64_t t = blockIdx.x;
  if (remap) t = (t & 7) * (gridDim.x >> 3) + (t >> 3);
  const int64_t blk = t % p.nblk;
  t /= p.nblk;
  const int64_t nt = t % n_tiles;
  t /= n_tiles;
  const int64_t mt = t % m_tiles;
  const int64_t split = t / m_tiles;
  const int64_t kb = p.partial ? split * p.k_chunk : 0;
  const int64_t ke = p.partial ? (kb + p.k_chunk < p.K ? kb + p.k_chunk : p.K) : p.K;
  const int64_t i0 = mt * TM, j0 = nt * TN;

  TA a;
  a.init(static_cast<const T*>(p.A) + blk * p.a_sb, i0, p.M, AM == 1 ? p.a_si : 1, 0, 0, p.a_sk,
         kb, ke);
  TB b;
  b.init(static_cast<const T*>(p.B) + blk * p.b_sb, j0, p.N, BMD == 1 ? p.b_sj : 1, p.b_sj_hi,
         BMD == 1 ? p.nsplit : 0, p.b_sk, kb, ke);

  f32x4 acc[FM][FN];
#pragma unroll
  for (int mi = 0; mi < FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (kb < ke) {
    a.load(kb);
    b.load(kb);
  }
  for (int64_t k0 = kb; k0 < ke; k0 += TK) {
    a.store(As, k0);
    b.store(Bs, k0);
    __syncthreads();
    if (k0 + TK < ke) {
      a.load(k0 + TK);
      b.load(k0 + TK);
    }
    if constexpr (C::kBf16) {
#pragma unroll
      for (int ks = 0; ks < TK; ks += 32) {
        bf16x8 fa[FM], fb[FN];
#pragma unroll
        for (int mi = 0; mi < FM; ++mi)
          fa[mi] = as_bf16x8(*reinterpret_cast<const u16x8*>(
              &As[C::rowoff((wm * FM + mi) * 16 + l15) + ks + 8 * lh]));
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
          fb[ni] = as_bf16x8(*reinterpret_cast<const u16x8*>(
              &Bs[C::rowoff((wn * FN + ni) * 16 + l15) + ks + 8 * lh]));
#pragma unroll
        for (int mi = 0; mi < FM; ++mi)
#pragma unroll
          for (int ni = 0; ni < FN; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
      }
    } else {
      // lane group lh supplies k = ks + 4*lh + j in the j-th of four MFMAs
      // (the same k on both operands), so one 16-byte LDS read per operand
      // feeds four products
#pragma unroll
      for (int ks = 0; ks < TK; ks += 16) {
        f32x4 fa[FM], fb[FN];
#pragma unroll
        for (int mi = 0; mi < FM; ++mi)
          fa[mi] = *reinterpret_cast<const f32x4*>(&As[C::rowoff((wm * FM + mi) * 16 + l15) + ks + 4 * lh]);
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
          fb[ni] = *reinterpret_cast<const f32x4*>(&Bs[C::rowoff((wn * FN + ni) * 16 + l15) + ks + 4 * lh]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int mi = 0; mi < FM; ++mi)
#pragma unroll
            for (int ni = 0; ni < FN; ++ni)
              acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[mi][j], fb[ni][j], acc[mi][ni], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // 16x16 result layout: lane holds rows 4*(lane/16)+v, column lane%16
#pragma unroll
  for (int ni = 0; ni < FN; ++ni) {
    const int64_t j = j0 + (wn * FN + ni) * 16 + l15;
    const int64_t joff = col_off(j, p.nsplit, p.c_sj_hi, p.c_sj);
#pragma unroll
    for (int mi = 0; mi < FM; ++mi)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t i = i0 + (wm * FM + mi) * 16 + 4 * lh + v;
        if (i < p.M && j < p.N) {
          float val = acc[mi][ni][v];
          if (p.partial) {
            p.partial[((split * p.nblk + blk) * p.M + i) * p.N + j] = val;
          } else {
            if (p.relu) val = val > 0.f ? val : 0.f;
            Io<T>::store(p.C, blk * p.c_sb + i * p.c_si + joff, val);
          }
        }
      }
  }
}

// keep v where m > 0 (ReLU derivative), element-wise on a 16-byte piece
template <typename T>
__device__ __forceinline__ u32x4 mask_piece(u32x4 v, u32x4 m) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (std::is_same<T, uint16_t>::value) {
      uint32_t keep = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t x = (m[i] >> (16 * h)) & 0xffffu;
        // bf16 > 0: sign clear, not zero, not NaN
        const bool pos = (x & 0x8000u) == 0 && x != 0 && x <= 0x7f80u;
        keep |= pos ? (0xffffu << (16 * h)) : 0u;
      }
      r[i] = v[i] & keep;
    } else {
      r[i] = __uint_as_float(m[i]) > 0.f ? v[i] : 0u;
    }
  }
  return r;
}

// dV rows from dY rows through LDS: each workgroup takes rpw whole rows,
// reads them with 16-byte loads (masking on the way), and writes the
// permuted rows with 16-byte stores. dV position o = g*q2o + p takes dY
// position p*b2 + g.
template <typename T>
__global__ __launch_bounds__(256) void dv_gather_lds_kernel(const T* __restrict__ dY,
                                                            const T* __restrict__ Ym,
                                                            T* __restrict__ dV, int64_t rows,
                                                            int64_t out, int64_t b2, int64_t q2o,
                                                            int rpw) {
  constexpr int VEC = 16 / static_cast<int>(sizeof(T));
  extern __shared__ __attribute__((aligned(16))) unsigned char dv_smem[];
  T* s = reinterpret_cast<T*>(dv_smem);
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * rpw;
  const int64_t nr = rows - row0 < rpw ? rows - row0 : rpw;
  const int64_t pieces = nr * out / VEC;
  const T* src = dY + row0 * out;
  const T* msk = Ym ? Ym + row0 * out : nullptr;
  for (int64_t e = threadIdx.x; e < pieces; e += 256) {
    u32x4 v = ld16(src + e * VEC);
    if (msk) v = mask_piece<T>(v, ld16(msk + e * VEC));
    *reinterpret_cast<u32x4*>(s + e * VEC) = v;
  }
  __syncthreads();
  T* dst = dV + row0 * out;
  for (int64_t e = threadIdx.x; e < pieces; e += 256) {
    const int64_t r = (e * VEC) / out, o0 = e * VEC - r * out;
    T vals[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const int64_t o = o0 + i;
      const int64_t g = o / q2o, pp = o - g * q2o;
      vals[i] = s[r * out + pp * b2 + g];
    }
    u32x4 w;
    __builtin_memcpy(&w, vals, sizeof(w));
    *reinterpret_cast<u32x4*>(dst + e * VEC) = w;
  }
}

// Element-wise fallback for rows that are too long for LDS or not a whole
// number of 16-byte pieces.
template <typename T>
__global__ __launch_bounds__(256) void dv_gather_kernel(const T* __restrict__ dY,
                                                        const T* __restrict__ Ym,
                                                        T* __restrict__ dV, int64_t rows,
                                                        int64_t out, int64_t b2, int64_t q2o) {
  const int64_t n = rows * out;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t b = e / out, o = e - b * out;
    const int64_t src = b * out + (o % q2o) * b2 + o / q2o;
    T v = dY[src];
    if (Ym && !(Io<T>::load(Ym, src) > 0.f)) v = T(0);
    dV[e] = v;
  }
}

// Tile shapes (TM x TN) and their wave grids
enum Shape { S128x128, S256x64, S256x32, S64x64, S32x32 };

Shape pick_shape(int64_t M, int64_t N) {
  if (M >= 256) {
    if (N > 64) return S128x128;
    if (N > 32) return S256x64;
    return S256x32;
  }
  if (M > 64 && N > 64) return S128x128;
  if (M > 32 || N > 32) return S64x64;
  return S32x32;
}

void shape_tiles(Shape s, int* tm, int* tn) {
  switch (s) {
    case S128x128: *tm = 128, *tn = 128; return;
    case S256x64: *tm = 256, *tn = 64; return;
    case S256x32: *tm = 256, *tn = 32; return;
    case S64x64: *tm = 64, *tn = 64; return;
    case S32x32: *tm = 32, *tn = 32; return;
  }
}

bool mode1_ok(int64_t s_contig, int64_t s_row, int64_t s_blk, int64_t kdim, int vec) {
  return s_contig == 1 && s_row % vec == 0 && s_blk % vec == 0 && kdim % vec == 0;
}
bool mode2_ok(int64_t s_contig, int64_t s_k, int64_t s_blk, int64_t rows, int vec) {
  return s_contig == 1 && s_k % vec == 0 && s_blk % vec == 0 && rows % vec == 0;
}

template <typename T, int AM, int BMD>
hipError_t launch_modes(const GemmArgs& a, Shape sh, dim3 g, int64_t mt, int64_t nt, int remap,
                        hipStream_t s) {
#define MONARCH_TILED(WM, WN, FM, FN) \
  hipLaunchKernelGGL((tiled_gemm_kernel<T, AM, BMD, WM, WN, FM, FN>), g, dim3(TT), 0, s, a, mt, nt, remap)
  switch (sh) {
    case S128x128: MONARCH_TILED(2, 2, 4, 4); break;
    case S256x64: MONARCH_TILED(4, 1, 4, 4); break;
    case S256x32: MONARCH_TILED(4, 1, 4, 2); break;
    case S64x64: MONARCH_TILED(2, 2, 2, 2); break;
    case S32x32: MONARCH_TILED(2, 2, 1, 1); break;
  }
#undef MONARCH_TILED
  return hipGetLastError();
}

}  // namespace

bool tiled_gemm_applicable(const GemmArgs& a, bool bf16) {
  const int vec = bf16 ? 8 : 4;
  if (a.M < 16 || a.N < 16 || a.K < 16) return false;  // tiny blocks: the generic kernel
  if (a.partial && (a.k_chunk % kSplitK != 0 || a.nsplit > 0)) return false;
  const bool a1 = mode1_ok(a.a_sk, a.a_si, a.a_sb, a.K, vec);
  const bool a2 = mode2_ok(a.a_si, a.a_sk, a.a_sb, a.M, vec);
  const bool b1 = a.nsplit > 0
                      ? (a.b_sk == 1 && a.b_sj % vec == 0 && a.b_sj_hi % vec == 0 &&
                         a.b_sb % vec == 0 && a.K % vec == 0)
                      : mode1_ok(a.b_sk, a.b_sj, a.b_sb, a.K, vec);
  const bool b2 = a.nsplit == 0 && mode2_ok(a.b_sj, a.b_sk, a.b_sb, a.N, vec);
  return (a1 || a2) && (b1 || b2);
}

hipError_t launch_tiled_gemm(const GemmArgs& a, bool bf16, hipStream_t s) {
  if (!tiled_gemm_applicable(a, bf16)) return hipErrorInvalidValue;
  const int vec = bf16 ? 8 : 4;
  const bool a1 = mode1_ok(a.a_sk, a.a_si, a.a_sb, a.K, vec);
  const bool b1 = a.nsplit > 0 || mode1_ok(a.b_sk, a.b_sj, a.b_sb, a.K, vec);
  const Shape sh = pick_shape(a.M, a.N);
  int tm, tn;
  shape_tiles(sh, &tm, &tn);
  const int64_t mt = (a.M + tm - 1) / tm, nt = (a.N + tn - 1) / tn;
  const int64_t grid = mt * nt * a.nblk * (a.partial ? a.splits : 1);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int remap = grid % 8 == 0 ? 1 : 0;
  const dim3 g(static_cast<unsigned>(grid));
  if (bf16) {
    if (a1 && b1) return launch_modes<uint16_t, 1, 1>(a, sh, g, mt, nt, remap, s);
    if (a1) return launch_modes<uint16_t, 1, 2>(a, sh, g, mt, nt, remap, s);
    if (b1) return launch_modes<uint16_t, 2, 1>(a, sh, g, mt, nt, remap, s);
    return launch_modes<uint16_t, 2, 2>(a, sh, g, mt, nt, remap, s);
  }
  if (a1 && b1) return launch_modes<float, 1, 1>(a, sh, g, mt, nt, remap, s);
  if (a1) return launch_modes<float, 1, 2>(a, sh, g, mt, nt, remap, s);
  if (b1) return launch_modes<float, 2, 1>(a, sh, g, mt, nt, remap, s);
  return launch_modes<float, 2, 2>(a, sh, g, mt, nt, remap, s);
}

hipError_t launch_gemm(const GemmArgs& a, bool bf16, hipStream_t s) {
  return tiled_gemm_applicable(a, bf16) ? launch_tiled_gemm(a, bf16, s)
                                        : launch_generic_gemm(a, bf16, s);
}

hipError_t launch_dv_gather(const void* dy, const void* ymask, void* dv, int64_t rows, int64_t out,
                            int64_t b2, int64_t q2o, bool bf16, hipStream_t s) {
  const int64_t n = rows * out;
  if (n <= 0) return hipSuccess;
  const int esz = bf16 ? 2 : 4, vec = 16 / esz;
  constexpr int64_t kLds = 32768;
  const int64_t row_bytes = out * esz;
  if (out % vec == 0 && row_bytes <= kLds) {
    const int rpw = static_cast<int>(kLds / row_bytes);
    const int64_t blocks = (rows + rpw - 1) / rpw;
    if (blocks <= 0x7fffffffLL) {
      const size_t lds = static_cast<size_t>(rpw) * row_bytes;
      if (bf16)
        hipLaunchKernelGGL(dv_gather_lds_kernel<uint16_t>, dim3(static_cast<unsigned>(blocks)),
                           dim3(256), lds, s, static_cast<const uint16_t*>(dy),
                           static_cast<const uint16_t*>(ymask), static_cast<uint16_t*>(dv), rows,
                           out, b2, q2o, rpw);
      else
        hipLaunchKernelGGL(dv_gather_lds_kernel<float>, dim3(static_cast<unsigned>(blocks)),
                           dim3(256), lds, s, static_cast<const float*>(dy),
                           static_cast<const float*>(ymask), static_cast<float*>(dv), rows, out,
                           b2, q2o, rpw);
      return hipGetLastError();
    }
  }
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (bf16)
    hipLaunchKernelGGL(dv_gather_kernel<uint16_t>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       s, static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(ymask),
                       static_cast<uint16_t*>(dv), rows, out, b2, q2o);
  else
    hipLaunchKernelGGL(dv_gather_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<const float*>(dy), static_cast<const float*>(ymask),
                       static_cast<float*>(dv), rows, out, b2, q2o);
  return hipGetLastError();
}

}  // namespace monarch
