// Device-side helpers shared by the HIP kernels of the MLA library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// bfloat16 is carried as its raw 16-bit pattern; conversions are explicit.
typedef uint16_t bf16;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16 v) {
  return __uint_as_float(((uint32_t)v) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (lo in bits 0..15), rounded to nearest, ties
// to even (one v_cvt_pk_bf16_f32 on gfx950; NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t r = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16 f32_to_bf16(float f) {
  return (bf16)(pack_bf16x2(f, 0.f) & 0xffffu);
}

// Storage-type traits: float or bf16.
template <typename T> struct St;
template <> struct St<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static float to_f(float v) { return v; }
  __device__ __forceinline__ static float from_f(float v) { return v; }
};
template <> struct St<bf16> {
  __device__ __forceinline__ static float load(const bf16* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static float to_f(bf16 v) { return bf16_to_f32(v); }
  __device__ __forceinline__ static bf16 from_f(float v) { return f32_to_bf16(v); }
};

template <typename T> __device__ __forceinline__ float ldf(const T* p) { return St<T>::to_f(*p); }
template <typename T> __device__ __forceinline__ void stf(T* p, float v) { *p = St<T>::from_f(v); }

__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace mla
