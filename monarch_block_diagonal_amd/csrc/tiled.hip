// Tiled strided batched GEMM for the generic Monarch path (gfx950).
//
// Contract: GemmArgs in kernels.h (a batch of independent block products at
// affine offsets, ReLU, bias and accumulation on the result, fp32
// batch-split partials, the optional column split), for operands whose
// elements are contiguous along one tile dimension:
//   A: K-contiguous (mode 1) or M-contiguous (mode 2),
//   B: K-contiguous (mode 1) or N-contiguous (mode 2).
// Every step of the Monarch product meets this once the saved intermediate
// is kept in stage 2's order and dY is gathered into block-major order (both
// arranged by the planner), so operand tiles move as 16-byte pieces.
//
// Workgroup: 256 threads = 4 waves in a WM x WN grid (512 threads = 8 waves
// for the bf16 256 x 256 and 256 x 192 tiles, 128 x 64 or 128 x 48 per wave:
// about half the operand bytes per product of the 128 x 128 tile); each
// wave owns FM x FN 16x16 MFMA tiles (bf16: v_mfma_f32_16x16x32_bf16, fp32:
// v_mfma_f32_16x16x4_f32; fp32 accumulation). K step: 64 (bf16) or 32
// (fp32). Both operand tiles sit in LDS as [row][k] with a 16-byte skew per
// 16 rows. A mode-1 piece is one 16-byte store; a mode-2 thread loads four
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


template <typename T>
struct Cfg {
  static constexpr bool kBf16 = std::is_same<T, uint16_t>::value;
  static constexpr int VEC = 16 / static_cast<int>(sizeof(T));  // elements per 16-byte piece
  static constexpr int TK = kBf16 ? 64 : 32;                     // K step
  static constexpr int LD = TK + VEC;                             // LDS row pitch (elements)
  // LDS offset of tile row r: a 144-byte pitch puts the 16 rows of a
  // fragment read on distinct bank groups, and a 16-byte skew per 16 rows
  // does the same for the transposed stores (rows 8 apart)
  static __device__ __host__ constexpr int rowoff(int r) { return r * LD + (r >> 4) * VEC; }
};

__device__ __forceinline__ void pin(u32x4& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ u32x4 ld16(const void* p) { return *static_cast<const u32x4*>(p); }
// 16 bytes at 4-byte alignment (global loads of this width need only
// dword alignment): fp32 operands whose blocks start off a 16-byte boundary
typedef uint32_t u32x4u __attribute__((ext_vector_type(4), aligned(4)));
__device__ __forceinline__ u32x4 ld16u(const void* p) {
  const u32x4u v = *static_cast<const u32x4u*>(p);
  return u32x4{v[0], v[1], v[2], v[3]};
}

// One operand tile (A: rows = M, B: rows = N) of ROWS x TK elements.
//   mode 1 (K-major units): unit = VEC consecutive k of one row;
//   mode 2 (row-major units): unit = four consecutive k of VEC consecutive rows.
// With `vec` a unit's VEC elements are one 16-byte load (the operand is
// contiguous along the unit with 16-byte aligned starts, and every limit is
// a multiple of VEC); otherwise they are loaded one by one with any strides.
// init() resolves each unit's row address once; elements past the row limit
// or the K range are loaded from a clamped in-range address and stored as
// zeros. An operand row sits at base + (r / ns)*hi + (r % ns)*lo (ns > 0,
// mode 1 only) or base + r*lo; `sk` is the K stride.
template <typename T, int MODE, int ROWS, bool EW, int SLOTS, int TT>
struct Tile {
  using C = Cfg<T>;
  static constexpr int VEC = C::VEC, TK = C::TK;
  static constexpr int UNITS = MODE == 1 ? ROWS * (TK / VEC) : (ROWS / VEC) * (TK / 4);
  static constexpr int NU = (UNITS + TT - 1) / TT;
  static constexpr int NR = MODE == 1 ? NU : 4 * NU;
  static constexpr int LDS = C::rowoff(ROWS);
  static_assert(ROWS % VEC == 0, "row pieces");

  const T* row[NU];   // address of the unit's first element at k = 0
  int nrow[NU];       // valid rows of the unit (mode 1: 0 or 1; mode 2: 0..VEC)
  int eclamp[NU];     // mode 2: largest row offset loads may use
  int64_t lo, sk, kb, ke;
  bool vec_;
  u32x4 reg[SLOTS][NR];   // K tiles in flight

  // without EW every operand of the launch moves as 16-byte pieces
  __device__ __forceinline__ bool vec() const { return EW ? vec_ : true; }

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
  __device__ __forceinline__ static u32x4 pack(const T (&v)[VEC]) {
    u32x4 r;
    __builtin_memcpy(&r, v, sizeof(r));
    return r;
  }

  // lim >= 1 rows are valid (callers skip the K loop when an operand has none)
  __device__ __forceinline__ void init(const T* base, int64_t r0, int64_t lim, int64_t lo_,
                                       int64_t hi, int64_t ns, int64_t sk_, int64_t kb_,
                                       int64_t ke_, bool vec_in) {
    lo = lo_, sk = sk_, kb = kb_, ke = ke_, vec_ = vec_in;
#pragma unroll
    for (int q = 0; q < NU; ++q) {
      const int64_t gr = r0 + unit_row(q);
      if constexpr (MODE == 1) {
        nrow[q] = gr < lim ? 1 : 0;
        eclamp[q] = 0;
        const int64_t r = gr < lim ? gr : 0;
        row[q] = base + (ns > 0 ? (r / ns) * hi + (r % ns) * lo : r * lo);
      } else {
        const int64_t nv = lim - gr;
        nrow[q] = nv <= 0 ? 0 : (nv >= VEC ? VEC : static_cast<int>(nv));
        const int64_t room = nv > 0 ? nv : lim;           // rows loads may touch
        eclamp[q] = room >= VEC ? VEC - 1 : static_cast<int>(room - 1);
        row[q] = base + (nv > 0 ? gr : 0) * lo;
      }
    }
  }

  template <int S>
  __device__ __forceinline__ void load(int64_t k0) {
#pragma unroll
    for (int q = 0; q < NU; ++q) {
      if (!active(q)) continue;
      const int k = unit_k(q);
      if constexpr (MODE == 1) {
        if (vec()) {
          int64_t gk = k0 + k;
          gk = gk < ke ? gk : kb;
          reg[S][q] = ld16(row[q] + gk);
        } else if (!C::kBf16 && sk == 1 && k0 + k + VEC <= ke) {
          // fp32, K-contiguous, the whole piece in range
          reg[S][q] = ld16u(row[q] + k0 + k);
        } else {
          T v[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            int64_t gk = k0 + k + e;
            gk = gk < ke ? gk : ke - 1;
            v[e] = row[q][gk * sk];
          }
          reg[S][q] = pack(v);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int64_t gk = k0 + k + i;
          gk = gk < ke ? gk : ke - 1;
          if (vec()) {
            reg[S][4 * q + i] = ld16(row[q] + gk * sk);
          } else if (!C::kBf16 && lo == 1 && nrow[q] == VEC) {
            // fp32, row-contiguous, all VEC rows valid
            reg[S][4 * q + i] = ld16u(row[q] + gk * sk);
          } else {
            T v[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[e] = row[q][(e < eclamp[q] ? e : eclamp[q]) * lo + gk * sk];
            reg[S][4 * q + i] = pack(v);
          }
        }
      }
    }
  }

  // keep element e of a loaded unit piece only where keep_e holds
  __device__ __forceinline__ static u32x4 mask_elems(u32x4 v, int nvalid_rows, bool kok_all,
                                                     int64_t kfirst, int64_t ke_) {
    T el[VEC];
    __builtin_memcpy(el, &v, sizeof(v));
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const bool keep = MODE == 1 ? (nvalid_rows > 0 && kfirst + e < ke_) : (e < nvalid_rows && kok_all);
      if (!keep) el[e] = T(0);
    }
    return pack(el);
  }

  template <int S>
  __device__ __forceinline__ void store(T* s, int64_t k0) {
#pragma unroll
    for (int q = 0; q < NU; ++q) {
      if (!active(q)) continue;
      const int r = unit_row(q), k = unit_k(q);
      if constexpr (MODE == 1) {
        pin(reg[S][q]);
        u32x4 v;
        if (vec()) {
          const bool keep = nrow[q] > 0 && k0 + k < ke;
          v = keep ? reg[S][q] : u32x4{0u, 0u, 0u, 0u};
        } else {
          v = mask_elems(reg[S][q], nrow[q], true, k0 + k, ke);
        }
        *reinterpret_cast<u32x4*>(s + C::rowoff(r) + k) = v;
      } else {
        u32x4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pin(reg[S][4 * q + i]);
          const bool kok = k0 + k + i < ke;
          if (vec())
            v[i] = (nrow[q] > 0 && kok) ? reg[S][4 * q + i] : u32x4{0u, 0u, 0u, 0u};
          else
            v[i] = mask_elems(reg[S][4 * q + i], nrow[q], kok, 0, 0);
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

// K tiles kept in flight in registers: two, or one for the 256-row tiles,
// whose A tile alone takes as many registers as two slots of the others; LDS
// buffers: two, or one for the 256 x 64 and 256 x 32 tiles (the 256 x 256
// tile keeps one register slot and two buffers).
template <int TM>
constexpr int kSlots = TM > 128 ? 1 : 2;
template <int TM, int TN>
constexpr int kBufs = TM > 128 && TN < 192 ? 1 : 2;

// Four consecutive elements of the I/O type as fp32 (8-byte bf16 or 16-byte
// fp32 accesses; offsets are multiples of four).
template <typename T> struct Vec4;
template <> struct Vec4<float> {
  static __device__ __forceinline__ f32x4 load(const void* p, int64_t i) {
    return *reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + i);
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, f32x4 v) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(p) + i) = v;
  }
};
template <> struct Vec4<uint16_t> {
  static __device__ __forceinline__ f32x4 load(const void* p, int64_t i) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p) + i);
    return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                 __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, f32x4 v) {
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p) + i) =
        u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
};

// Writes a workgroup's TM x TN result tile the way GemmArgs asks (plain,
// 4-wide, fp32 partial, or with accumulation, bias, ReLU and the column
// split). acc holds wave (wm, wn)'s FM x FN 16x16 MFMA tiles.
template <typename T, int WM, int WN, int FM, int FN>
__device__ __forceinline__ void write_tile(const GemmArgs& p, const f32x4 (&acc)[FM][FN],
                                           int64_t blk, int64_t split, int64_t i0, int64_t j0,
                                           int wm, int wn, int l15, int lh) {
  constexpr int TM = WM * FM * 16, TN = WN * FN * 16;
  // 16x16 result layout: lane holds rows 4*(lane/16)+v, column lane%16
  const int64_t cblk = blk * p.c_sb;
  // a whole tile of stores that keep every column (the common case) skips
  // the per-element range checks and steps row offsets by the row stride;
  // bias (one load per column) and ReLU fold in
  const bool plain = !p.partial && !p.accum && p.c_cols < 0 && i0 + TM <= p.M && j0 + TN <= p.N;
  // offset of this lane's first row (v = 0 of tile row 0)
  const int64_t rb = (i0 + wm * FM * 16 + 4 * lh) * p.c_si;
  if (p.cvec && plain) {
    const int u = l15 & 3;
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) {
      const int64_t jb = j0 + (wn * FN + ni) * 16 + (l15 & ~3);
      const int64_t cpos = cblk + (p.nsplit > 0 ? col_off(jb, p.nsplit, p.c_sj_hi, 1) : jb);
      T* c = static_cast<T*>(p.C) + rb + u * p.c_si + cpos;
      const f32x4 bv = p.bias ? Vec4<T>::load(p.bias, cpos) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mi = 0; mi < FM; ++mi) {
        f32x4 o = quad_transpose4(acc[mi][ni], u) + bv;
        if (p.relu) {
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = o[e] > 0.f ? o[e] : 0.f;
        }
        Vec4<T>::store(c, mi * 16 * p.c_si, o);
      }
    }
    return;
  }
  if (p.partial && i0 + TM <= p.M && j0 + TN <= p.N) {
    float* P = p.partial + ((split * p.nblk + blk) * p.M + i0 + wm * FM * 16 + 4 * lh) * p.N + j0 +
               wn * FN * 16 + l15;
#pragma unroll
    for (int ni = 0; ni < FN; ++ni)
#pragma unroll
      for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int v = 0; v < 4; ++v) P[(mi * 16 + v) * p.N + ni * 16] = acc[mi][ni][v];
    return;
  }
  if (plain) {
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) {
      const int64_t j = j0 + (wn * FN + ni) * 16 + l15;
      const int64_t cpos = cblk + col_off(j, p.nsplit, p.c_sj_hi, p.c_sj);
      T* c = static_cast<T*>(p.C) + rb + cpos;
      const float bv = p.bias ? Io<T>::load(p.bias, cpos) : 0.f;
#pragma unroll
      for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float o = acc[mi][ni][v] + bv;
          if (p.relu) o = o > 0.f ? o : 0.f;
          Io<T>::store(c, (mi * 16 + v) * p.c_si, o);
        }
    }
    return;
  }
  if (p.cvec) {
    // a 4x4 transpose within each quad of lanes (columns 4c..4c+3) leaves
    // lane 4c+u with row 4*(lane/16)+u, columns 4c..4c+3: one 4-element
    // load/store per row instead of four single elements. In rotation r
    // lane u sends its row (u - r) & 3 and receives, by a DPP quad
    // permutation (lane u reads lane (u + r) & 3), row u of column
    // (u + r) & 3; the selections are two-level on the bits of a
    // loop-invariant lane index, so they stay selects, not branches.
    const int u = l15 & 3;
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) {
      const int64_t jb = j0 + (wn * FN + ni) * 16 + (l15 & ~3);
      // with a column split the four columns stay within one piece
      const int64_t cpos = cblk + (p.nsplit > 0 ? col_off(jb, p.nsplit, p.c_sj_hi, 1) : jb);
#pragma unroll
      for (int mi = 0; mi < FM; ++mi) {
        f32x4 o = quad_transpose4(acc[mi][ni], u);
        const int64_t i = i0 + (wm * FM + mi) * 16 + 4 * lh + u;
        if (i < p.M && jb < p.N && (p.c_cols < 0 || cpos < p.c_cols)) {
          const int64_t off = i * p.c_si + cpos;
          if (p.accum) o += Vec4<T>::load(p.C, off);
          if (p.bias) o += Vec4<T>::load(p.bias, cpos);
          if (p.relu) {
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = o[e] > 0.f ? o[e] : 0.f;
          }
          Vec4<T>::store(p.C, off, o);
        }
      }
    }
    return;
  }
#pragma unroll
  for (int ni = 0; ni < FN; ++ni) {
    const int64_t j = j0 + (wn * FN + ni) * 16 + l15;
    const int64_t cpos = cblk + col_off(j, p.nsplit, p.c_sj_hi, p.c_sj);   // in-row offset
#pragma unroll
    for (int mi = 0; mi < FM; ++mi)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t i = i0 + (wm * FM + mi) * 16 + 4 * lh + v;
        if (i < p.M && j < p.N) {
          float val = acc[mi][ni][v];
          if (p.partial) {
            p.partial[((split * p.nblk + blk) * p.M + i) * p.N + j] = val;
          } else if (p.c_cols < 0 || cpos < p.c_cols) {
            if (p.accum) val += Io<T>::load(p.C, i * p.c_si + cpos);
            if (p.bias) val += Io<T>::load(p.bias, cpos);
            if (p.relu) val = val > 0.f ? val : 0.f;
            Io<T>::store(p.C, i * p.c_si + cpos, val);
          }
        }
      }
  }
}

// A whole tile of contiguous bf16 output (columns unit-stride, or runs of a
// column split that are whole 16-byte pieces) can leave through LDS once the
// K loop is done (ct: TM x TN elements of free LDS). Written straight from the
// MFMA layout, a store instruction covers 16 rows with 32 bytes each; from LDS
// every instruction writes whole 2*TN-byte row segments, and those whole
// lines leave with non-temporal stores (9% faster on the GPT-2 stage-1
// forward; the strided two-byte stores of the other paths need L2 to merge
// the blocks' lines and stay plain). Tile row r keeps its 16-byte chunk c at
// c ^ (r & 7). Returns false, having done nothing, when the tile does not
// qualify; every thread of the workgroup must call it.
template <int WM, int WN, int FM, int FN>
__device__ __forceinline__ bool write_tile_staged(const GemmArgs& p, const f32x4 (&acc)[FM][FN],
                                                  int64_t blk, int64_t i0, int64_t j0, int wm,
                                                  int wn, int l15, int lh, int tid, uint16_t* ct) {
  constexpr int TM = WM * FM * 16, TN = WN * FN * 16, NT = WM * WN * 64;
  static_assert(TN % 64 == 0, "the chunk swizzle needs whole groups of 8 chunks");
  const bool staged = !p.partial && !p.accum && p.c_cols < 0 && p.c_sj == 1 &&
                      i0 + TM <= p.M && j0 + TN <= p.N && p.c_si % 8 == 0 && p.c_sb % 8 == 0 &&
                      (p.nsplit == 0 || (p.nsplit % 8 == 0 && p.c_sj_hi % 8 == 0)) &&
                      (reinterpret_cast<uintptr_t>(p.C) & 15) == 0;
  if (!staged) return false;
  __syncthreads();
  constexpr int NCH = TN / 8;   // 16-byte chunks per tile row
  {
    const int u = l15 & 3;
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) {
      const int jc = (wn * FN + ni) * 16 + (l15 & ~3);   // first of this lane's 4 columns
      const f32x4 bv = p.bias ? Vec4<uint16_t>::load(p.bias, blk * p.c_sb +
                                                    (p.nsplit > 0 ? col_off(j0 + jc, p.nsplit, p.c_sj_hi, 1) : j0 + jc))
                              : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mi = 0; mi < FM; ++mi) {
        f32x4 o = quad_transpose4(acc[mi][ni], u) + bv;
        if (p.relu) {
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = o[e] > 0.f ? o[e] : 0.f;
        }
        const int r = (wm * FM + mi) * 16 + 4 * lh + u;
        *reinterpret_cast<u32x2*>(&ct[r * TN + (((jc >> 3) ^ (r & 7)) << 3) + (jc & 7)]) =
            u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      }
    }
  }
  __syncthreads();
  uint16_t* C = static_cast<uint16_t*>(p.C) + blk * p.c_sb;
#pragma unroll 4
  for (int id = tid; id < TM * NCH; id += NT) {
    const int r = id / NCH, c = id - r * NCH;
    const int64_t j = j0 + 8 * c;
    const int64_t col = p.nsplit > 0 ? col_off(j, p.nsplit, p.c_sj_hi, 1) : j;
    __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(&ct[r * TN + ((c ^ (r & 7)) << 3)]),
                                reinterpret_cast<u32x4*>(C + (i0 + r) * p.c_si + col));
  }
  return true;
}

template <typename T, int AM, int BMD, int WM, int WN, int FM, int FN, bool EW>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(2)))
void tiled_gemm_kernel(GemmArgs p, int64_t m_tiles,
                                                        int64_t n_tiles, int remap, int avec,
                                                        int bvec) {
  using C = Cfg<T>;
  constexpr int TM = WM * FM * 16, TN = WN * FN * 16, TK = C::TK;
  static_assert(WM * WN == 4 || WM * WN == 8, "four or eight waves");
  constexpr int TT = WM * WN * 64;
  // the element-wise variants keep one K tile in registers: their per-element
  // loads and masks need the room of the second slot
  constexpr int SL = EW ? 1 : kSlots<TM>, LB = kBufs<TM, TN>;
  using TA = Tile<T, AM, TM, EW, SL, TT>;
  using TB = Tile<T, BMD, TN, EW, SL, TT>;
  // one LDS array for both operands' buffers, so that a bf16 output tile
  // can be staged in it after the K loop
  __shared__ __attribute__((aligned(16))) T smem[LB * (TA::LDS + TB::LDS)];
  T (*As)[TA::LDS] = reinterpret_cast<T (*)[TA::LDS]>(smem);
  T (*Bs)[TB::LDS] = reinterpret_cast<T (*)[TB::LDS]>(smem + LB * TA::LDS);
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
  int64_t ke = p.partial ? (kb + p.k_chunk < p.K ? kb + p.k_chunk : p.K) : p.K;
  // zero padding: this block's valid K range and B columns
  if (p.k_lim >= 0) {
    const int64_t kv = p.k_lim - blk * p.k_lim_bs;
    ke = ke < kv ? ke : kv;
  }
  int64_t nlim = p.N;
  if (p.n_lim >= 0) {
    const int64_t nv = p.n_lim - blk * p.n_lim_bs;
    nlim = nlim < nv ? nlim : nv;
  }
  if (nlim <= 0 || ke < kb) ke = kb;   // nothing to sum: the K loop is skipped
  const int64_t i0 = mt * TM, j0 = nt * TN;

  TA a;
  a.init(static_cast<const T*>(p.A) + blk * p.a_sb, i0, p.M, p.a_si, 0, 0, p.a_sk, kb, ke,
         avec != 0);
  TB b;
  b.init(static_cast<const T*>(p.B) + blk * p.b_sb, j0, nlim > 0 ? nlim : 1, p.b_sj, p.b_sj_hi,
         BMD == 1 ? p.nsplit : 0, p.b_sk, kb, ke, bvec != 0);

  f32x4 acc[FM][FN];
#pragma unroll
  for (int mi = 0; mi < FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  // K tile t sits in register slot t % SL and LDS buffer t % SL.
  //  * One slot (256-row tiles): step t stores slot 0 to LDS, reloads it with
  //    tile t + 1, multiplies, and waits twice.
  //  * Two slots: step t multiplies buffer t % 2 while it stores tile t + 1
  //    (slot (t + 1) % 2) into the other buffer and reloads that slot with
  //    tile t + 3; one barrier per step, and a load has two steps to land.
  //  * One slot, two buffers (256 x 256): step t multiplies buffer t % 2,
  //    stores tile t + 1 from the slot into the other buffer and reloads the
  //    slot with tile t + 2; one barrier per step, and a load has one
  //    multiply of eight waves to land.
  const int64_t nsteps = kb < ke ? (ke - kb + TK - 1) / TK : 0;
  auto mult = [&](const T* as, const T* bs) {
    if constexpr (C::kBf16) {
#pragma unroll
      for (int ks = 0; ks < TK; ks += 32) {
        bf16x8 fa[FM], fb[FN];
#pragma unroll
        for (int mi = 0; mi < FM; ++mi)
          fa[mi] = as_bf16x8(*reinterpret_cast<const u16x8*>(
              &as[C::rowoff((wm * FM + mi) * 16 + l15) + ks + 8 * lh]));
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
          fb[ni] = as_bf16x8(*reinterpret_cast<const u16x8*>(
              &bs[C::rowoff((wn * FN + ni) * 16 + l15) + ks + 8 * lh]));
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
          fa[mi] = *reinterpret_cast<const f32x4*>(&as[C::rowoff((wm * FM + mi) * 16 + l15) + ks + 4 * lh]);
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
          fb[ni] = *reinterpret_cast<const f32x4*>(&bs[C::rowoff((wn * FN + ni) * 16 + l15) + ks + 4 * lh]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int mi = 0; mi < FM; ++mi)
#pragma unroll
            for (int ni = 0; ni < FN; ++ni)
              acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[mi][j], fb[ni][j], acc[mi][ni], 0, 0, 0);
      }
    }
  };
  if constexpr (SL == 1 && LB == 2) {
    if (nsteps > 0) {
      a.template load<0>(kb);
      b.template load<0>(kb);
      a.template store<0>(As[0], kb);
      b.template store<0>(Bs[0], kb);
      if (nsteps > 1) {
        a.template load<0>(kb + TK);
        b.template load<0>(kb + TK);
      }
      __syncthreads();
    }
    auto step = [&](auto buf, int64_t t) {
      constexpr int S = decltype(buf)::value, S1 = 1 - S;
      const int64_t k1 = kb + (t + 1) * TK;
      mult(As[S], Bs[S]);
      if (t + 1 < nsteps) {
        a.template store<0>(As[S1], k1);
        b.template store<0>(Bs[S1], k1);
        if (t + 2 < nsteps) {
          a.template load<0>(k1 + TK);
          b.template load<0>(k1 + TK);
        }
      }
      __syncthreads();
    };
    for (int64_t t = 0; t < nsteps; t += 2) {
      step(std::integral_constant<int, 0>{}, t);
      if (t + 1 < nsteps) step(std::integral_constant<int, 1>{}, t + 1);
    }
  } else if constexpr (SL == 1) {
    if (nsteps > 0) {
      a.template load<0>(kb);
      b.template load<0>(kb);
    }
    for (int64_t t = 0; t < nsteps; ++t) {
      const int64_t k0 = kb + t * TK;
      a.template store<0>(As[0], k0);
      b.template store<0>(Bs[0], k0);
      __syncthreads();
      if (t + 1 < nsteps) {
        a.template load<0>(k0 + TK);
        b.template load<0>(k0 + TK);
      }
      mult(As[0], Bs[0]);
      __syncthreads();
    }
  } else {
    if (nsteps > 0) {
      a.template load<0>(kb);
      b.template load<0>(kb);
      if (nsteps > 1) {
        a.template load<1>(kb + TK);
        b.template load<1>(kb + TK);
      }
      a.template store<0>(As[0], kb);
      b.template store<0>(Bs[0], kb);
      if (nsteps > 2) {
        a.template load<0>(kb + 2 * TK);
        b.template load<0>(kb + 2 * TK);
      }
      __syncthreads();
    }
    auto step = [&](auto buf, int64_t t) {
      constexpr int S = decltype(buf)::value, S1 = 1 - S;
      const int64_t k1 = kb + (t + 1) * TK;
      mult(As[S], Bs[S]);
      if (t + 1 < nsteps) {
        a.template store<S1>(As[S1], k1);
        b.template store<S1>(Bs[S1], k1);
        if (t + 3 < nsteps) {
          a.template load<S1>(k1 + 2 * TK);
          b.template load<S1>(k1 + 2 * TK);
        }
      }
      __syncthreads();
    };
    for (int64_t t = 0; t < nsteps; t += 2) {
      step(std::integral_constant<int, 0>{}, t);
      if (t + 1 < nsteps) step(std::integral_constant<int, 1>{}, t + 1);
    }
  }

  if constexpr (C::kBf16 && TM >= 128 && TN % 64 == 0 && LB * (TA::LDS + TB::LDS) >= TM * TN) {
    if (write_tile_staged<WM, WN, FM, FN>(p, acc, blk, i0, j0, wm, wn, l15, lh, tid, smem)) return;
  }
  write_tile<T, WM, WN, FM, FN>(p, acc, blk, split, i0, j0, wm, wn, l15, lh);
}

// --------------------------------------------------------------------------
// Pipelined variant: bf16, both operands K-contiguous with 16-byte aligned
// pieces, the 256 x 256 and 256 x 192 tiles (8 waves, 128 x 64 or 128 x 48
// per wave).
// --------------------------------------------------------------------------
// At these tile sizes the register-staged kernel above has room for one K
// tile in flight, so each load has one multiply step to land. Here K tiles
// of 32 go from global memory straight into LDS (global_load_lds_dwordx4: a
// wave's 64 pieces land in 1 KB of LDS in lane order), PS stages deep: a
// tile has PS - 1 multiply steps to land and takes no registers. A stage
// holds 256 rows of A and 256 rows of B (the 192-wide tile loads 64 rows it
// does not use) as 64-byte rows of four 16-byte pieces; piece q of row r
// sits at position q ^ ((r >> 2) & 3), so the 16 rows of a fragment read
// fall on distinct banks. Each step waits for this wave's loads of its tile
// (vmcnt) and for its previous LDS reads, meets the other waves at a bare
// s_barrier (a workgroup fence would also wait for the loads of the later
// tiles), issues the loads of the tile PS - 1 steps ahead into the stage
// the previous step read, and multiplies. Rows past M or N are loaded from
// the last valid row and their results are not stored; the launcher checks
// that every K range is a whole number of tiles and that zero padding cuts
// no block.
constexpr int PS = 4;    // LDS stages
constexpr int PK = 32;   // K per stage

#define MONARCH_GPTR(p) ((__attribute__((address_space(1))) void*)(p))
#define MONARCH_LPTR(p) ((__attribute__((address_space(3))) void*)(p))
// s_waitcnt: vector memory count <= n, LDS count 0, export count untouched
#define MONARCH_WAIT_VM_LDS(n) (((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4))

// zero-padding limits are allowed when they cut no block (the last block's
// valid range still covers K, or N)
bool pipe_ok(const GemmArgs& a) {
  const int64_t last = a.nblk - 1;
  const bool kfull = a.k_lim < 0 || a.k_lim - last * a.k_lim_bs >= a.K;
  const bool nfull = a.n_lim < 0 || a.n_lim - last * a.n_lim_bs >= a.N;
  return a.K % PK == 0 && kfull && nfull && (!a.partial || a.k_chunk % PK == 0);
}

template <int FN>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void pipe_gemm_kernel(GemmArgs p, int64_t m_tiles, int64_t n_tiles, int remap) {
  constexpr int WM = 2, WN = 4, FM = 8;
  constexpr int TM = WM * FM * 16, TN = WN * FN * 16;
  static_assert(TM == 256 && TN <= 256, "tile");
  __shared__ __attribute__((aligned(16))) u32x4 lds[PS][2][256 * 4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  // load instruction i of this wave: tile rows (2*wave + i)*16 + lane/4,
  // LDS position lane % 4, global piece (lane % 4) ^ ((row >> 2) & 3)
  const uint16_t* ap[2];
  const uint16_t* bp[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (2 * wave + i) * 16 + (lane >> 2);
    const int q = (lane & 3) ^ ((r >> 2) & 3);
    const int64_t ar = i0 + r < p.M ? i0 + r : p.M - 1;
    const int64_t br = j0 + r < p.N ? j0 + r : p.N - 1;
    ap[i] = static_cast<const uint16_t*>(p.A) + blk * p.a_sb + ar * p.a_si + 8 * q;
    bp[i] = static_cast<const uint16_t*>(p.B) + blk * p.b_sb +
            (p.nsplit > 0 ? (br / p.nsplit) * p.b_sj_hi + (br % p.nsplit) * p.b_sj : br * p.b_sj) +
            8 * q;
  }

  f32x4 acc[FM][FN];
#pragma unroll
  for (int mi = 0; mi < FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t nsteps = kb < ke ? (ke - kb) / PK : 0;
  auto issue = [&](int64_t s) {
    const int st = static_cast<int>(s % PS);
    const int64_t k0 = kb + s * PK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_global_load_lds(MONARCH_GPTR(ap[i] + k0),
                                       MONARCH_LPTR(&lds[st][0][(2 * wave + i) * 64]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(MONARCH_GPTR(bp[i] + k0),
                                       MONARCH_LPTR(&lds[st][1][(2 * wave + i) * 64]), 16, 0, 0);
    }
  };
  // fragment rows: (tile base multiple of 16) + l15, so the swizzle is lane-constant
  const int sw = lh ^ ((l15 >> 2) & 3);
  auto mult = [&](const u32x4* as, const u32x4* bs) {
    bf16x8 fa[FM], fb[FN];
#pragma unroll
    for (int mi = 0; mi < FM; ++mi) {
      const u32x4 v = as[((wm * FM + mi) * 16 + l15) * 4 + sw];
      __builtin_memcpy(&fa[mi], &v, sizeof(v));
    }
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) {
      const u32x4 v = bs[((wn * FN + ni) * 16 + l15) * 4 + sw];
      __builtin_memcpy(&fb[ni], &v, sizeof(v));
    }
#pragma unroll
    for (int mi = 0; mi < FM; ++mi)
#pragma unroll
      for (int ni = 0; ni < FN; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
  };

  for (int64_t s = 0; s < PS - 1 && s < nsteps; ++s) issue(s);
  for (int64_t s = 0; s < nsteps; ++s) {
    // tiles issued after tile s (four loads each per wave)
    const int64_t later = nsteps - 1 - s < PS - 2 ? nsteps - 1 - s : PS - 2;
    asm volatile("" ::: "memory");
    if (later >= 2)
      __builtin_amdgcn_s_waitcnt(MONARCH_WAIT_VM_LDS(8));
    else if (later == 1)
      __builtin_amdgcn_s_waitcnt(MONARCH_WAIT_VM_LDS(4));
    else
      __builtin_amdgcn_s_waitcnt(MONARCH_WAIT_VM_LDS(0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (s + PS - 1 < nsteps) issue(s + PS - 1);
    const int st = static_cast<int>(s % PS);
    mult(lds[st][0], lds[st][1]);
  }
  if (!write_tile_staged<WM, WN, FM, FN>(p, acc, blk, i0, j0, wm, wn, l15, lh, tid,
                                         reinterpret_cast<uint16_t*>(&lds[0][0][0])))
    write_tile<uint16_t, WM, WN, FM, FN>(p, acc, blk, split, i0, j0, wm, wn, l15, lh);
}
#undef MONARCH_GPTR
#undef MONARCH_LPTR
#undef MONARCH_WAIT_VM_LDS

// keep v where m > 0 (ReLU derivative), element-wise on a 16-byte piece
template <typename T>
__device__ __forceinline__ u32x4 mask_piece(u32x4 v, u32x4 m) {
  if constexpr (std::is_same<T, uint16_t>::value) {
    return relu_mask_bf16(v, m);
  } else {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __uint_as_float(m[i]) > 0.f ? v[i] : 0u;
    return r;
  }
}

// dV rows from dY rows through LDS: each workgroup takes rpw whole rows,
// reads them with 16-byte loads (masking on the way), and writes the
// permuted rows with 16-byte stores. dV position o = g*q2o + p takes dY
// position p*b2 + g when that is below out (truncated outputs: 0).
template <typename T>
__global__ __launch_bounds__(256) void dv_gather_lds_kernel(const T* __restrict__ dY,
                                                            const T* __restrict__ Ym,
                                                            T* __restrict__ dV, int64_t rows,
                                                            int64_t out, int64_t b2, int64_t q2o,
                                                            int rpw) {
  constexpr int VEC = 16 / static_cast<int>(sizeof(T));
  extern __shared__ __attribute__((aligned(16))) unsigned char dv_smem[];
  T* s = reinterpret_cast<T*>(dv_smem);
  const int64_t oext = b2 * q2o;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * rpw;
  const int64_t nr = rows - row0 < rpw ? rows - row0 : rpw;
  const int64_t in_pieces = nr * out / VEC, out_pieces = nr * oext / VEC;
  const T* src = dY + row0 * out;
  const T* msk = Ym ? Ym + row0 * out : nullptr;
  for (int64_t e = threadIdx.x; e < in_pieces; e += 256) {
    u32x4 v = ld16(src + e * VEC);
    if (msk) v = mask_piece<T>(v, ld16(msk + e * VEC));
    *reinterpret_cast<u32x4*>(s + e * VEC) = v;
  }
  __syncthreads();
  T* dst = dV + row0 * oext;
  // offsets inside the staged rows fit 32 bits (at most 32 KB of them); one
  // division per piece, then (g, p) steps along the piece
  const uint32_t oe = static_cast<uint32_t>(oext), q = static_cast<uint32_t>(q2o);
  const uint32_t nb = static_cast<uint32_t>(b2), ou = static_cast<uint32_t>(out);
  for (uint32_t e = threadIdx.x; e < static_cast<uint32_t>(out_pieces); e += 256) {
    const uint32_t r = (e * VEC) / oe, o0 = e * VEC - r * oe;
    uint32_t g = o0 / q, pp = o0 - g * q;
    const T* srow = s + r * ou;
    T vals[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const uint32_t so = pp * nb + g;
      vals[i] = so < ou ? srow[so] : T(0);
      if (++pp == q) pp = 0, ++g;
    }
    u32x4 w;
    __builtin_memcpy(&w, vals, sizeof(w));
    *reinterpret_cast<u32x4*>(dst + static_cast<int64_t>(e) * VEC) = w;
  }
}

// Element-wise form for rows that are too long for LDS or not a whole
// number of 16-byte pieces.
template <typename T>
__global__ __launch_bounds__(256) void dv_gather_kernel(const T* __restrict__ dY,
                                                        const T* __restrict__ Ym,
                                                        T* __restrict__ dV, int64_t rows,
                                                        int64_t out, int64_t b2, int64_t q2o) {
  const int64_t oext = b2 * q2o;
  const int64_t n = rows * oext;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t b = e / oext, o = e - b * oext;
    const int64_t so = (o % q2o) * b2 + o / q2o;
    T v = T(0);
    if (so < out) {
      const int64_t src = b * out + so;
      v = dY[src];
      if (Ym && !(Io<T>::load(Ym, src) > 0.f)) v = T(0);
    }
    dV[e] = v;
  }
}

// partial[c][p*b2 + g] = sum over rows of chunk c of dV[b, g*q2o + p]: one
// thread per dV column, rows in increasing order (deterministic).
template <typename T>
__global__ __launch_bounds__(256) void bias_partials_kernel(const T* __restrict__ dV,
                                                            float* __restrict__ partial,
                                                            int64_t rows, int64_t chunk,
                                                            int64_t out, int64_t b2, int64_t q2o) {
  const int64_t oext = b2 * q2o;
  const int64_t col = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t c = blockIdx.y;
  if (col >= oext) return;
  const int64_t g = col / q2o, pp = col - g * q2o, o = pp * b2 + g;
  if (o >= out) return;
  const int64_t r0 = c * chunk, r1 = r0 + chunk < rows ? r0 + chunk : rows;
  // eight rows' loads in flight, added in row order
  float acc = 0.f;
  const T* src = dV + col;
  int64_t b = r0;
  for (; b + 8 <= r1; b += 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = Io<T>::load(src, (b + i) * oext);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += v[i];
  }
  for (; b < r1; ++b) acc += Io<T>::load(src, b * oext);
  partial[c * out + o] = acc;
}

// Tile shapes (TM x TN) and their wave grids
enum Shape { S256x256, S256x192, S128x128, S256x64, S256x32, S64x64, S32x32 };

// 256 x 256 for bf16 products of at least 256 x 256, 256 x 192 for those
// 129 to 192 columns wide (batch splits of such products are sized for these
// tiles by the planner)
Shape pick_shape(int64_t M, int64_t N, bool bf16) {
  if (bf16 && M >= 256 && N >= 256) return S256x256;
  if (bf16 && M >= 256 && N > 128 && N <= 192) return S256x192;
  if (M >= 256) {
    if (N > 64) return S128x128;
    if (N > 32) return S256x64;
    return S256x32;
  }
  if (M <= 32) return S32x32;
  if (M > 64 && N > 64) return S128x128;
  if (M > 32 || N > 32) return S64x64;
  return S32x32;
}

// Operands loaded element by element take the smaller tiles: the 256-row
// tiles of the element-wise variant would not fit in 256 VGPRs per lane.
Shape ew_shape(Shape s) {
  switch (s) {
    case S256x256:
    case S256x192: return S128x128;
    case S256x64: return S64x64;
    default: return s;
  }
}

void shape_tiles(Shape s, int* tm, int* tn) {
  switch (s) {
    case S256x256: *tm = 256, *tn = 256; return;
    case S256x192: *tm = 256, *tn = 192; return;
    case S128x128: *tm = 128, *tn = 128; return;
    case S256x64: *tm = 256, *tn = 64; return;
    case S256x32: *tm = 256, *tn = 32; return;
    case S64x64: *tm = 64, *tn = 64; return;
    case S32x32: *tm = 32, *tn = 32; return;
  }
}

bool lim_ok(int64_t lim, int64_t lim_bs, int vec) {
  return lim < 0 || (lim % vec == 0 && lim_bs % vec == 0);
}

template <typename T, int AM, int BMD>
hipError_t launch_modes(const GemmArgs& a, Shape sh, dim3 g, int64_t mt, int64_t nt, int remap,
                        int avec, int bvec, hipStream_t s) {
#define MONARCH_TILED(WM, WN, FM, FN)                                                         \
  if (avec && bvec)                                                                             \
    hipLaunchKernelGGL((tiled_gemm_kernel<T, AM, BMD, WM, WN, FM, FN, false>), g,              \
                       dim3(WM * WN * 64), 0, s, a, mt, nt, remap, 1, 1);                        \
  else                                                                                          \
    hipLaunchKernelGGL((tiled_gemm_kernel<T, AM, BMD, WM, WN, FM, FN, true>), g,               \
                       dim3(WM * WN * 64), 0, s, a, mt, nt, remap, avec, bvec)
  // shapes that ew_shape() keeps away from the element-wise loads
#define MONARCH_TILED_VEC(WM, WN, FM, FN)                                                     \
  if (!(avec && bvec)) return hipErrorInvalidValue;                                            \
  hipLaunchKernelGGL((tiled_gemm_kernel<T, AM, BMD, WM, WN, FM, FN, false>), g,                \
                     dim3(WM * WN * 64), 0, s, a, mt, nt, remap, 1, 1)
  switch (sh) {
    case S256x256:
      if constexpr (std::is_same<T, uint16_t>::value && AM == 1 && BMD == 1) {
        if (avec && bvec && pipe_ok(a)) {
          hipLaunchKernelGGL(pipe_gemm_kernel<4>, g, dim3(512), 0, s, a, mt, nt, remap);
          break;
        }
      }
      if constexpr (std::is_same<T, uint16_t>::value) {
        MONARCH_TILED_VEC(2, 4, 8, 4);
      } else {
        return hipErrorInvalidValue;
      }
      break;
    case S256x192:
      if constexpr (std::is_same<T, uint16_t>::value && AM == 1 && BMD == 1) {
        if (avec && bvec && pipe_ok(a)) {
          hipLaunchKernelGGL(pipe_gemm_kernel<3>, g, dim3(512), 0, s, a, mt, nt, remap);
          break;
        }
      }
      if constexpr (std::is_same<T, uint16_t>::value) {
        MONARCH_TILED_VEC(2, 4, 8, 3);
      } else {
        return hipErrorInvalidValue;
      }
      break;
    case S128x128: MONARCH_TILED(2, 2, 4, 4); break;
    case S256x64: MONARCH_TILED_VEC(4, 1, 4, 4); break;
    case S256x32: MONARCH_TILED(4, 1, 4, 2); break;
    case S64x64: MONARCH_TILED(2, 2, 2, 2); break;
    case S32x32: MONARCH_TILED(2, 2, 1, 1); break;
  }
#undef MONARCH_TILED
#undef MONARCH_TILED_VEC
  return hipGetLastError();
}

int64_t iabs(int64_t v) { return v < 0 ? -v : v; }

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, bool bf16, hipStream_t s) {
  if (const int bdm = bd_mode(a, bf16)) return launch_bd(a, bdm, s);
  if (const int skm = skinny_mode(a, bf16)) return launch_skinny(a, skm, bf16, s);
  const int vec = bf16 ? 8 : 4;
  // A: K-major units when K is its faster dimension, row-major otherwise
  const int am = a.a_sk == 1 ? 1 : (a.a_si == 1 ? 2 : (iabs(a.a_sk) <= iabs(a.a_si) ? 1 : 2));
  const bool klim = lim_ok(a.k_lim, a.k_lim_bs, vec);
  const bool avec = am == 1 ? (a.a_sk == 1 && a.a_si % vec == 0 && a.a_sb % vec == 0 &&
                               a.K % vec == 0 && klim)
                            : (a.a_si == 1 && a.a_sk % vec == 0 && a.a_sb % vec == 0 &&
                               a.M % vec == 0);
  // B: the column split needs K-major units
  const int bm = a.nsplit > 0 ? 1
                              : (a.b_sk == 1 ? 1 : (a.b_sj == 1 ? 2 : (iabs(a.b_sk) <= iabs(a.b_sj) ? 1 : 2)));
  const bool bvec = bm == 1 ? (a.b_sk == 1 && a.b_sj % vec == 0 &&
                               (a.nsplit == 0 || a.b_sj_hi % vec == 0) && a.b_sb % vec == 0 &&
                               a.K % vec == 0 && klim)
                            : (a.b_sj == 1 && a.b_sk % vec == 0 && a.b_sb % vec == 0 &&
                               a.N % vec == 0 && lim_ok(a.n_lim, a.n_lim_bs, vec));
  if (a.partial && (a.k_chunk % kSplitK != 0 || a.nsplit > 0)) return hipErrorInvalidValue;
  GemmArgs g4 = a;
  g4.cvec = !a.partial && (a.nsplit == 0 || (a.nsplit % 4 == 0 && a.c_sj_hi % 4 == 0)) &&
            a.c_sj == 1 && a.c_sb % 4 == 0 && a.c_si % 4 == 0 &&
            a.N % 4 == 0 && (a.c_cols < 0 || a.c_cols % 4 == 0);
  Shape sh = avec && bvec ? pick_shape(a.M, a.N, bf16) : ew_shape(pick_shape(a.M, a.N, bf16));
  int tm, tn;
  shape_tiles(sh, &tm, &tn);
  // An unsplit product whose large tiles would leave most CUs idle (fewer
  // than 128 workgroups, each with a long K loop) takes 64 x 64 tiles: the
  // recommender MLP's 1000 x 2500 -> 256 blocks went from 64 to 256
  // workgroups, 0.195 -> 0.070 ms. Batch-split products are sized by the
  // planner and keep their tiles.
  if (!a.partial && tm * tn > 64 * 64 &&
      ((a.M + tm - 1) / tm) * ((a.N + tn - 1) / tn) * a.nblk < 128) {
    sh = S64x64;
    shape_tiles(sh, &tm, &tn);
  }
  const int64_t mt = (a.M + tm - 1) / tm, nt = (a.N + tn - 1) / tn;
  const int64_t grid = mt * nt * a.nblk * (a.partial ? a.splits : 1);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int remap = grid % 8 == 0 ? 1 : 0;
  const dim3 g(static_cast<unsigned>(grid));
  const int av = avec ? 1 : 0, bv = bvec ? 1 : 0;
  if (bf16) {
    if (am == 1 && bm == 1) return launch_modes<uint16_t, 1, 1>(g4, sh, g, mt, nt, remap, av, bv, s);
    if (am == 1) return launch_modes<uint16_t, 1, 2>(g4, sh, g, mt, nt, remap, av, bv, s);
    if (bm == 1) return launch_modes<uint16_t, 2, 1>(g4, sh, g, mt, nt, remap, av, bv, s);
    return launch_modes<uint16_t, 2, 2>(g4, sh, g, mt, nt, remap, av, bv, s);
  }
  if (am == 1 && bm == 1) return launch_modes<float, 1, 1>(g4, sh, g, mt, nt, remap, av, bv, s);
  if (am == 1) return launch_modes<float, 1, 2>(g4, sh, g, mt, nt, remap, av, bv, s);
  if (bm == 1) return launch_modes<float, 2, 1>(g4, sh, g, mt, nt, remap, av, bv, s);
  return launch_modes<float, 2, 2>(g4, sh, g, mt, nt, remap, av, bv, s);
}

hipError_t launch_dv_gather(const void* dy, const void* ymask, void* dv, int64_t rows, int64_t out,
                            int64_t b2, int64_t q2o, bool bf16, hipStream_t s) {
  const int64_t oext = b2 * q2o;
  if (rows <= 0 || oext <= 0) return hipSuccess;
  // unmasked and untruncated: each row's [q2o][b2] becomes [b2][q2o], the
  // axis swap (padded LDS tiles, several rows per workgroup)
  if (!ymask && out == oext) return launch_swap(dy, dv, rows, q2o, 1, b2, bf16, s);
  const int esz = bf16 ? 2 : 4, vec = 16 / esz;
  constexpr int64_t kLds = 32768;
  const int64_t row_bytes = out * esz;
  if (out % vec == 0 && oext % vec == 0 && row_bytes <= kLds) {
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
  int64_t blocks = (rows * oext + 255) / 256;
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

hipError_t launch_bias_partials(const void* dv, float* partial, int64_t rows, int64_t chunk,
                                int64_t chunks, int64_t out, int64_t b2, int64_t q2o, bool bf16,
                                hipStream_t s) {
  const int64_t oext = b2 * q2o;
  if (rows <= 0 || chunks <= 0) return hipSuccess;
  const int64_t gx = (oext + 255) / 256;
  if (gx > 0x7fffffffLL || chunks > 65535) return hipErrorInvalidConfiguration;
  const dim3 g(static_cast<unsigned>(gx), static_cast<unsigned>(chunks));
  if (bf16)
    hipLaunchKernelGGL(bias_partials_kernel<uint16_t>, g, dim3(256), 0, s,
                       static_cast<const uint16_t*>(dv), partial, rows, chunk, out, b2, q2o);
  else
    hipLaunchKernelGGL(bias_partials_kernel<float>, g, dim3(256), 0, s,
                       static_cast<const float*>(dv), partial, rows, chunk, out, b2, q2o);
  return hipGetLastError();
}

}  // namespace monarch
