// Shared device helpers for the Monarch kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace monarch {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bfloat16 is carried as its raw 16-bit pattern.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 with the hardware conversion (v_cvt_pk_bf16_f32): round to
// nearest even, NaN stays NaN. Branch-free, so it adds no control flow to
// the kernels' main loops.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const __bf16 r = static_cast<__bf16>(f);
  uint16_t u;
  __builtin_memcpy(&u, &r, sizeof(u));
  return u;
}

// two fp32 -> packed pair of bf16 (low half = a), one conversion instruction
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  const bf16x2 r = __builtin_convertvector(v, bf16x2);
  uint32_t u;
  __builtin_memcpy(&u, &r, sizeof(u));
  return u;
}

template <typename T> struct Io;
template <> struct Io<float> {
  static __device__ __forceinline__ float load(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
};
template <> struct Io<uint16_t> {
  static __device__ __forceinline__ float load(const void* p, int64_t i) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
  }
};

__device__ __forceinline__ bf16x8 as_bf16x8(u16x8 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
}

// Offset of output column j under the optional column split of GemmArgs
// (kernels.h): j*lo, or (j / ns)*hi + (j % ns)*lo when ns > 0.
__device__ __forceinline__ int64_t col_off(int64_t j, int64_t ns, int64_t hi, int64_t lo) {
  return ns > 0 ? (j / ns) * hi + (j % ns) * lo : j * lo;
}

// Keeps the bf16 halves of v whose mask half is > 0 (the ReLU derivative,
// taken as 0 at 0): sign clear, not zero, not NaN.
__device__ __forceinline__ u32x4 relu_mask_bf16(u32x4 v, u32x4 m) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t keep = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t x = (m[i] >> (16 * h)) & 0xffffu;
      const bool pos = (x & 0x8000u) == 0 && x != 0 && x <= 0x7f80u;
      keep |= pos ? (0xffffu << (16 * h)) : 0u;
    }
    r[i] = v[i] & keep;
  }
  return r;
}

// 4x8 transpose of bf16 in registers: in[i] holds elements (i, e = 0..7);
// out[e] gets elements (i = 0..3, e) packed into 8 bytes.
__device__ __forceinline__ void transpose4x8(const u32x4 (&in)[4], u32x2 (&out)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    out[2 * k][0] = (in[0][k] & 0xffffu) | (in[1][k] << 16);
    out[2 * k][1] = (in[2][k] & 0xffffu) | (in[3][k] << 16);
    out[2 * k + 1][0] = (in[0][k] >> 16) | (in[1][k] & 0xffff0000u);
    out[2 * k + 1][1] = (in[2][k] >> 16) | (in[3][k] & 0xffff0000u);
  }
}

// 4x4 transpose of 32-bit elements: out[e][i] = in[i][e].
__device__ __forceinline__ void transpose4x4(const u32x4 (&in)[4], u32x4 (&out)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = u32x4{in[0][e], in[1][e], in[2][e], in[3][e]};
}

}  // namespace monarch
