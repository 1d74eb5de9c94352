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

// 8x8 transpose of bf16 in registers: in[i] holds elements (i, e = 0..7);
// out[e] gets elements (i = 0..7, e).
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
  u32x2 lo[8], hi[8];
  transpose4x8(*reinterpret_cast<const u32x4(*)[4]>(&in[0]), lo);
  transpose4x8(*reinterpret_cast<const u32x4(*)[4]>(&in[4]), hi);
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = u32x4{lo[e][0], lo[e][1], hi[e][0], hi[e][1]};
}

// 4x4 transpose of 32-bit elements: out[e][i] = in[i][e].
__device__ __forceinline__ void transpose4x4(const u32x4 (&in)[4], u32x4 (&out)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = u32x4{in[0][e], in[1][e], in[2][e], in[3][e]};
}

// Element k of a lane's four values, chosen on the bits of k (selects,
// not branches, when k differs between lanes).
__device__ __forceinline__ float pick4(const f32x4& v, int k) {
  const float lo = (k & 1) ? v[1] : v[0];
  const float hi = (k & 1) ? v[3] : v[2];
  return (k & 2) ? hi : lo;
}
template <int CTRL>
__device__ __forceinline__ float quad_read(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
// 4x4 transpose within a quad of lanes: lane u holds rows 0..3 of column u
// of a 4x4 block and returns row u, columns 0..3. Rotation r moves, by a
// quad permutation where lane u reads lane (u + r) & 3, the value each lane
// holds for the lane that reads it.
__device__ __forceinline__ f32x4 quad_transpose4(const f32x4& in, int u) {
  const float g0 = pick4(in, u);
  const float g1 = quad_read<0x39>(pick4(in, (u - 1) & 3));   // quad_perm [1,2,3,0]
  const float g2 = quad_read<0x4e>(pick4(in, (u - 2) & 3));   // quad_perm [2,3,0,1]
  const float g3 = quad_read<0x93>(pick4(in, (u - 3) & 3));   // quad_perm [3,0,1,2]
  // g_r is column (u + r) & 3
  f32x4 o;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int r = (c - u) & 3;
    const float lo = (r & 1) ? g1 : g0;
    const float hi = (r & 1) ? g3 : g2;
    o[c] = (r & 2) ? hi : lo;
  }
  return o;
}

}  // namespace monarch
