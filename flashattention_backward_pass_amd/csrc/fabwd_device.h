// Device-side helpers shared by the gfx950 kernels of the backward library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fabwd {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 storage is a 16-bit pattern; arithmetic is always float32.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round-to-nearest-even float32 -> bf16 (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Element access for the two storage types.
template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <>
struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i].bits); }
  static __device__ __forceinline__ void store(bf16_t* p, int64_t i, float v) { p[i].bits = f32_to_bf16(v); }
};

// Hardware 2^x (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh(x / c) from the identity tanh(y) = 1 - 2 / (e^(2y) + 1), with
// k = 2 log2(e) / c precomputed so there is no division per element:
// e^(2x/c) = 2^(k x).  Odd-correct and saturating at both ends: 2^(k x)
// overflows to inf for large x (tanh -> 1) and underflows to 0 for very
// negative x (tanh -> -1).  Absolute error a few ulp of 1.
__device__ __forceinline__ float tanh_scaled(float x, float k) {
  const float e = fast_exp2(k * x);
  return fmaf(-2.0f, __builtin_amdgcn_rcpf(e + 1.0f), 1.0f);
}

__device__ __forceinline__ float wave_xor_sum(float v, int width) {
  for (int off = width >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, width);
  return v;
}
__device__ __forceinline__ float wave_xor_max(float v, int width) {
  for (int off = width >> 1; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, width));
  return v;
}

// fp32 add into global memory with the hardware float atomic (no CAS loop).
__device__ __forceinline__ void atomic_add_f32(float* p, float v) { unsafeAtomicAdd(p, v); }

}  // namespace fabwd
