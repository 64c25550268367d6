// Device helpers shared by the MLA kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

typedef uint16_t bf16;  // bfloat16 bit pattern (storage type)

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;   // MFMA A/B operand
typedef __attribute__((ext_vector_type(4))) short short4_t;     // transpose-read result
typedef __attribute__((ext_vector_type(16))) float f32x16;      // 32x32 MFMA accumulator
typedef __attribute__((ext_vector_type(4))) float f32x4;        // 16x16 MFMA accumulator
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

#define LDS_AS __attribute__((address_space(3)))

__device__ __forceinline__ float bf2f(bf16 x) { return __uint_as_float((uint32_t)x << 16); }

// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ bf16 f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (bf16)0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16)(u >> 16);
}

// Two floats -> packed pair of bf16 (low half = a), nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

template <typename T> __device__ __forceinline__ float ld(const T* p);
template <> __device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld<bf16>(const bf16* p) { return bf2f(*p); }

template <typename T> __device__ __forceinline__ void st(T* p, float v);
template <> __device__ __forceinline__ void st<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void st<bf16>(bf16* p, float v) { *p = f2bf(v); }

// RoPE angle of pair i at position pos: pos * base^(-2i/d_rope), formed in
// double so that positions in the tens of thousands keep their low bits; the
// caller takes sin/cos in double as well (few values per call).
__device__ __forceinline__ double rope_angle(int pos, int i, int d_rope, float base) {
  return (double)pos * pow((double)base, -2.0 * (double)i / (double)d_rope);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace mla
