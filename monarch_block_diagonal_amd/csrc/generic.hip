// Small helper kernels of the Monarch library (gfx950): the fixed-order
// reduction of batch-split gradient partial sums, axis swaps of batches of
// 3-D arrays and a zero fill.
//
// The weight gradients of both block-diagonal factors are sums over the
// batch (each block's gradient is its output gradient transposed times its
// input, summed over rows); the GEMM kernels write one fp32 partial per batch
// chunk and the reduction below adds the chunks in increasing order, so the
// result does not depend on scheduling.
#include "common.h"
#include "kernels.h"

namespace monarch {
namespace {

// Elements [0, a.n) of the flattened index space reduce a's partials, the
// next b.n elements b's, the rest c's.
template <typename T>
__global__ __launch_bounds__(256) void reduce_partials_kernel(ReduceArgs a, ReduceArgs b,
                                                              ReduceArgs c) {
  const int64_t total = a.n + b.n + c.n;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    const bool in_a = e < a.n, in_b = !in_a && e < a.n + b.n;
    const float* part = in_a ? a.partial : (in_b ? b.partial : c.partial);
    void* out = in_a ? a.out : (in_b ? b.out : c.out);
    const int64_t n = in_a ? a.n : (in_b ? b.n : c.n);
    const int64_t splits = in_a ? a.splits : (in_b ? b.splits : c.splits);
    const int64_t i = in_a ? e : (in_b ? e - a.n : e - a.n - b.n);
    // eight chunks' loads in flight, added in chunk order
    float s = 0.f;
    int64_t k = 0;
    for (; k + 8 <= splits; k += 8) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = part[(k + j) * n + i];
#pragma unroll
      for (int j = 0; j < 8; ++j) s += v[j];
    }
    for (; k < splits; ++k) s += part[k * n + i];
    Io<T>::store(out, i, s);
  }
}

// The same with four consecutive elements per thread (every n a multiple of
// 4): 16-byte partial loads, eight chunks in flight, the same chunk order
// for every element.
template <typename T>
__global__ __launch_bounds__(256) void reduce_partials4_kernel(ReduceArgs a, ReduceArgs b,
                                                               ReduceArgs c) {
  const int64_t total = (a.n + b.n + c.n) / 4;
  for (int64_t e4 = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e4 < total;
       e4 += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t e = 4 * e4;
    const bool in_a = e < a.n, in_b = !in_a && e < a.n + b.n;
    const float* part = in_a ? a.partial : (in_b ? b.partial : c.partial);
    void* out = in_a ? a.out : (in_b ? b.out : c.out);
    const int64_t n = in_a ? a.n : (in_b ? b.n : c.n);
    const int64_t splits = in_a ? a.splits : (in_b ? b.splits : c.splits);
    const int64_t i = in_a ? e : (in_b ? e - a.n : e - a.n - b.n);
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
    int64_t k = 0;
    for (; k + 8 <= splits; k += 8) {
      f32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = *reinterpret_cast<const f32x4*>(part + (k + j) * n + i);
#pragma unroll
      for (int j = 0; j < 8; ++j) s += v[j];
    }
    for (; k < splits; ++k) s += *reinterpret_cast<const f32x4*>(part + k * n + i);
#pragma unroll
    for (int q = 0; q < 4; ++q) Io<T>::store(out, i + q, s[q]);
  }
}

// Axis swaps out[b][c][m][a] = in[b][a][m][c] of batches of A x M x C
// arrays (the transposes and the layout changes between the rounds of the
// k-factor layer).
//
// Whole arrays through LDS (A*M*C elements fit): the array is read with
// 16-byte pieces and written as runs of consecutive a, 16-byte pieces when
// A allows, so both sides move whole lines however small A, M and C are.
// The LDS copy has one pad word per 64 words: the reads of a piece's
// elements step by M*C elements, which is often a multiple of 256 bytes.
template <typename T>
__device__ __forceinline__ int swap_pos(int i) {
  constexpr int EPW = 4 / sizeof(T);   // elements per 4-byte word
  return i + (i / (64 * EPW)) * EPW;
}
template <typename T>
constexpr int swap_lds_elems(int n) {
  return n + (n / (64 * (4 / static_cast<int>(sizeof(T)))) + 1) * (4 / static_cast<int>(sizeof(T)));
}

// out + v (accumulating swaps), in fp32, rounded once to the I/O type
__device__ __forceinline__ float add_io(float v, float o) { return v + o; }
__device__ __forceinline__ uint16_t add_io(uint16_t v, uint16_t o) {
  return f32_to_bf16(bf16_to_f32(v) + bf16_to_f32(o));
}
template <typename T>
__device__ __forceinline__ u32x4 add_piece(u32x4 v, u32x4 o) {
  T a[16 / sizeof(T)], b[16 / sizeof(T)];
  __builtin_memcpy(a, &v, 16);
  __builtin_memcpy(b, &o, 16);
#pragma unroll
  for (int e = 0; e < static_cast<int>(16 / sizeof(T)); ++e) a[e] = add_io(a[e], b[e]);
  u32x4 r;
  __builtin_memcpy(&r, a, 16);
  return r;
}

// A workgroup takes `per` consecutive arrays (the last one may take fewer),
// so that small arrays still give each workgroup a few KB to move. With
// `accum` the swapped values are added to what `out` holds.
template <typename T>
__global__ __launch_bounds__(256) void swap_lds_kernel(const T* __restrict__ in,
                                                      T* __restrict__ out, int A, int M, int C,
                                                      int vec, int64_t rows, int per, int accum) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* s = reinterpret_cast<T*>(smem);
  constexpr int V = 16 / sizeof(T);
  const int na = A * M * C;
  const int64_t a0 = static_cast<int64_t>(blockIdx.x) * per;
  const int cnt = rows - a0 < per ? static_cast<int>(rows - a0) : per;
  const int n = na * cnt;
  const int64_t base = a0 * na;
  const T* src = in + base;
  T* dst = out + base;
  const int tid = threadIdx.x;
  // vector pieces go U at a time per thread, every load issued before the
  // first wait
  constexpr int U = 4;
  const int nq = n / V;
  if (vec) {
    // a piece never straddles a pad (64*EPW is a multiple of V); its words
    // are stored one by one (the padded position is only word-aligned)
    for (int q0 = tid; q0 < nq; q0 += 256 * U) {
      u32x4 v[U];
#pragma unroll
      for (int j = 0; j < U; ++j)
        if (q0 + 256 * j < nq) v[j] = reinterpret_cast<const u32x4*>(src)[q0 + 256 * j];
#pragma unroll
      for (int j = 0; j < U; ++j)
        if (q0 + 256 * j < nq) {
          uint32_t* w = reinterpret_cast<uint32_t*>(s + swap_pos<T>((q0 + 256 * j) * V));
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = v[j][e];
        }
    }
  } else {
    for (int i = tid; i < n; i += 256) s[swap_pos<T>(i)] = src[i];
  }
  __syncthreads();
  if (vec) {
    // output piece o = V consecutive a of one (c, m) of array k
    for (int q0 = tid; q0 < nq; q0 += 256 * U) {
      u32x4 old[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        old[j] = u32x4{0u, 0u, 0u, 0u};
        if (accum && q0 + 256 * j < nq) old[j] = reinterpret_cast<const u32x4*>(dst)[q0 + 256 * j];
      }
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int q = q0 + 256 * j;
        if (q >= nq) continue;
        const int k = (q * V) / na, o = q * V - k * na;
        const int a0 = o % A, cm = o / A, m = cm % M, c = cm / M;
        T v[V];
#pragma unroll
        for (int e = 0; e < V; ++e) v[e] = s[swap_pos<T>(k * na + ((a0 + e) * M + m) * C + c)];
        u32x4 r;
        __builtin_memcpy(&r, v, sizeof(r));
        if (accum) r = add_piece<T>(r, old[j]);
        reinterpret_cast<u32x4*>(dst)[q] = r;
      }
    }
  } else {
    for (int oo = tid; oo < n; oo += 256) {
      const int k = oo / na, o = oo - k * na;
      const int a = o % A, cm = o / A, m = cm % M, c = cm / M;
      const T v = s[swap_pos<T>(k * na + (a * M + m) * C + c)];
      dst[oo] = accum ? add_io(v, dst[oo]) : v;
    }
  }
}

// Rows of A x 4 two-byte elements (M = 1, C = 4, A a multiple of 8) swapped
// to 4 x A in registers: a lane loads one 16-byte piece (positions 2k and
// 2k+1, all four c; the lanes of a wave read 1 KB contiguous), packs it into
// one 32-bit word per c (the two positions side by side), and a 4 x 4
// transpose within its quad of lanes (DPP moves, bit-exact) gives lane c of
// the quad the words of c for the quad's 8 consecutive positions: one
// 16-byte store, and 16 quads of a wave write 256-byte runs per c. No LDS.
// A quad's four pieces lie in one row (A/2 pieces per row, a multiple of 4)
// and quads are in or out of range as a whole, so the transpose runs with
// all four lanes of a quad active. A workgroup covers 1024 consecutive
// pieces: each thread takes up to four of them, 256 apart, loading all of
// them first.
__global__ __launch_bounds__(256) void swap_c4_kernel(const u32x4* __restrict__ in,
                                                      u32x4* __restrict__ out, int64_t rows,
                                                      int64_t A) {
  constexpr int U = 4;
  const int64_t ppr = A / 2;   // pieces per row
  const int64_t total = rows * ppr;
  const int u = threadIdx.x & 3;
  const int64_t p0 = static_cast<int64_t>(blockIdx.x) * 256 * U + threadIdx.x;
  u32x4 v[U];
#pragma unroll
  for (int j = 0; j < U; ++j)
    if (p0 + 256 * j < total) v[j] = __builtin_nontemporal_load(in + p0 + 256 * j);
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int64_t p = p0 + 256 * j;
    if (p >= total) continue;
    // words of c: (position 2k, c) in the low half, (2k + 1, c) in the high half
    f32x4 w;
    w[0] = __uint_as_float((v[j][0] & 0xffffu) | (v[j][2] << 16));
    w[1] = __uint_as_float((v[j][0] >> 16) | (v[j][2] & 0xffff0000u));
    w[2] = __uint_as_float((v[j][1] & 0xffffu) | (v[j][3] << 16));
    w[3] = __uint_as_float((v[j][1] >> 16) | (v[j][3] & 0xffff0000u));
    const f32x4 o = quad_transpose4(w, u);   // lane u: c = u, quad lanes' words in order
    const int64_t row = p / ppr, q = (p - row * ppr) >> 2;
    const u32x4 r{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                  __float_as_uint(o[3])};
    // element offset row*4A + u*A + 8q, in 16-byte pieces
    __builtin_nontemporal_store(r, out + row * ppr + u * (A / 8) + q);
  }
}

// Larger arrays: 32 x 32 (a, c) tiles of one (b, m) through LDS; reads run
// along c and writes along a.
template <typename T>
__global__ __launch_bounds__(256) void swap_tiled_kernel(const T* __restrict__ in,
                                                        T* __restrict__ out, int64_t A, int64_t M,
                                                        int64_t C, int64_t tiles_a,
                                                        int64_t tiles_c, int accum) {
  __shared__ T t[32][33];
  int64_t bid = blockIdx.x;
  const int64_t tc = bid % tiles_c;
  bid /= tiles_c;
  const int64_t ta = bid % tiles_a;
  bid /= tiles_a;
  const int64_t m = bid % M, b = bid / M;
  const T* src = in + b * A * M * C + m * C;    // (a, c) at a*M*C + c
  T* dst = out + b * A * M * C + m * A;         // (c, a) at c*M*A + a
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    const int64_t a = ta * 32 + i, c = tc * 32 + tx;
    if (a < A && c < C) t[i][tx] = src[a * M * C + c];
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int64_t c = tc * 32 + i, a = ta * 32 + tx;
    if (c < C && a < A) dst[c * M * A + a] = accum ? add_io(t[tx][i], dst[c * M * A + a]) : t[tx][i];
  }
}

__global__ __launch_bounds__(256) void zero_kernel(uint16_t* p, int64_t n) {
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * 256)
    p[e] = 0;
}

}  // namespace

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(bytes / 2);
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<uint16_t*>(p), n);
  return hipGetLastError();
}

hipError_t launch_swap(const void* in, void* out, int64_t rows, int64_t A, int64_t M, int64_t C,
                       bool bf16, hipStream_t s, bool accum) {
  const int acc = accum ? 1 : 0;
  if (rows <= 0 || A <= 0 || M <= 0 || C <= 0) return hipSuccess;
  if (bf16 && !accum && M == 1 && C == 4 && A % 8 == 0 &&
      (reinterpret_cast<uintptr_t>(in) & 15) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
    const int64_t quads = rows * (A / 2) / 4;   // whole quads of pieces
    const int64_t blocks = (rows * (A / 2) + 1023) / 1024;
    if (quads > 0 && blocks <= 0x7fffffffLL) {
      hipLaunchKernelGGL(swap_c4_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                         static_cast<const u32x4*>(in), static_cast<u32x4*>(out), rows, A);
      return hipGetLastError();
    }
  }
  const int64_t esz = bf16 ? 2 : 4, V = 16 / esz, n = A * M * C;
  constexpr int64_t kLds = 49 * 1024;
  // arrays per workgroup: about 4K elements of them (fewer, larger
  // workgroups lose more than they save on bigger arrays)
  const int64_t per = n < 4096 ? (4096 / n < rows ? 4096 / n : rows) : 1;
  const int64_t chunk = n * per;
  const int64_t lds_elems =
      chunk < (int64_t(1) << 20) ? (bf16 ? swap_lds_elems<uint16_t>(static_cast<int>(chunk))
                                         : swap_lds_elems<float>(static_cast<int>(chunk)))
                                 : chunk;
  const int64_t groups = (rows + per - 1) / per;
  if (lds_elems * esz <= kLds && groups <= 0x7fffffffLL) {
    const int vec = n % V == 0 && A % V == 0 ? 1 : 0;
    const size_t lds = static_cast<size_t>(lds_elems * esz);
    const dim3 g(static_cast<unsigned>(groups));
    if (bf16)
      hipLaunchKernelGGL(swap_lds_kernel<uint16_t>, g, dim3(256), lds, s,
                         static_cast<const uint16_t*>(in), static_cast<uint16_t*>(out),
                         static_cast<int>(A), static_cast<int>(M), static_cast<int>(C), vec, rows,
                         static_cast<int>(per), acc);
    else
      hipLaunchKernelGGL(swap_lds_kernel<float>, g, dim3(256), lds, s,
                         static_cast<const float*>(in), static_cast<float*>(out),
                         static_cast<int>(A), static_cast<int>(M), static_cast<int>(C), vec, rows,
                         static_cast<int>(per), acc);
    return hipGetLastError();
  }
  const int64_t ta = (A + 31) / 32, tc = (C + 31) / 32;
  const int64_t grid = rows * M * ta * tc;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (bf16)
    hipLaunchKernelGGL(swap_tiled_kernel<uint16_t>, dim3(static_cast<unsigned>(grid)), dim3(256),
                       0, s, static_cast<const uint16_t*>(in), static_cast<uint16_t*>(out), A, M,
                       C, ta, tc, acc);
  else
    hipLaunchKernelGGL(swap_tiled_kernel<float>, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                       s, static_cast<const float*>(in), static_cast<float*>(out), A, M, C, ta,
                       tc, acc);
  return hipGetLastError();
}

hipError_t launch_reduce_partials(const ReduceArgs& a, const ReduceArgs& b, const ReduceArgs& c,
                                  bool bf16, hipStream_t s) {
  const int64_t n = a.n + b.n + c.n;
  if (n <= 0) return hipSuccess;
  // partial buffers are 256-byte aligned workspace regions
  if (a.n % 4 == 0 && b.n % 4 == 0 && c.n % 4 == 0) {
    int64_t blocks = (n / 4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (bf16)
      hipLaunchKernelGGL(reduce_partials4_kernel<uint16_t>, dim3(static_cast<unsigned>(blocks)),
                         dim3(256), 0, s, a, b, c);
    else
      hipLaunchKernelGGL(reduce_partials4_kernel<float>, dim3(static_cast<unsigned>(blocks)),
                         dim3(256), 0, s, a, b, c);
    return hipGetLastError();
  }
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (bf16)
    hipLaunchKernelGGL(reduce_partials_kernel<uint16_t>, dim3(static_cast<unsigned>(blocks)),
                       dim3(256), 0, s, a, b, c);
  else
    hipLaunchKernelGGL(reduce_partials_kernel<float>, dim3(static_cast<unsigned>(blocks)),
                       dim3(256), 0, s, a, b, c);
  return hipGetLastError();
}

}  // namespace monarch
