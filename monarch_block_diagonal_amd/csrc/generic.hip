// Small helper kernels of the Monarch library (gfx950): the fixed-order
// reduction of batch-split gradient partial sums, a per-row transpose and a
// zero fill.
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

// 32 x 32 tiles through LDS: reads and writes run along rows of 32.
template <typename T>
__global__ __launch_bounds__(256) void row_transpose_kernel(const T* __restrict__ in,
                                                            T* __restrict__ out, int64_t R,
                                                            int64_t C, int64_t tiles_r,
                                                            int64_t tiles_c) {
  __shared__ T t[32][33];
  int64_t bid = blockIdx.x;
  const int64_t tcol = bid % tiles_c;
  bid /= tiles_c;
  const int64_t trow = bid % tiles_r;
  const int64_t b = bid / tiles_r;
  const T* src = in + b * R * C;
  T* dst = out + b * R * C;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    const int64_t r = trow * 32 + i, c = tcol * 32 + tx;
    if (r < R && c < C) t[i][tx] = src[r * C + c];
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int64_t c = tcol * 32 + i, r = trow * 32 + tx;
    if (c < C && r < R) dst[c * R + r] = t[tx][i];
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

hipError_t launch_row_transpose(const void* in, void* out, int64_t rows, int64_t R, int64_t C,
                                bool bf16, hipStream_t s) {
  if (rows <= 0 || R <= 0 || C <= 0) return hipSuccess;
  const int64_t tr = (R + 31) / 32, tc = (C + 31) / 32;
  const int64_t grid = rows * tr * tc;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (bf16)
    hipLaunchKernelGGL(row_transpose_kernel<uint16_t>, dim3(static_cast<unsigned>(grid)), dim3(256),
                       0, s, static_cast<const uint16_t*>(in), static_cast<uint16_t*>(out), R, C,
                       tr, tc);
  else
    hipLaunchKernelGGL(row_transpose_kernel<float>, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                       s, static_cast<const float*>(in), static_cast<float*>(out), R, C, tr, tc);
  return hipGetLastError();
}

hipError_t launch_reduce_partials(const ReduceArgs& a, const ReduceArgs& b, const ReduceArgs& c,
                                  bool bf16, hipStream_t s) {
  const int64_t n = a.n + b.n + c.n;
  if (n <= 0) return hipSuccess;
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
