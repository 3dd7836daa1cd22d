// Device-side helpers shared by the KDA kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

// Element types of the token tensors.
struct Bf16 {
  using storage = uint16_t;
  static constexpr int bytes = 2;
};
struct F32 {
  using storage = float;
  static constexpr int bytes = 4;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float load_scalar(const uint16_t* p, long i) { return bf16_bits_to_f32(p[i]); }
__device__ __forceinline__ float load_scalar(const float* p, long i) { return p[i]; }
__device__ __forceinline__ void store_scalar(uint16_t* p, long i, float x) { p[i] = f32_to_bf16_bits(x); }
__device__ __forceinline__ void store_scalar(float* p, long i, float x) { p[i] = x; }

// Input maps of the fused prologue, in fp32.
//   softplus(x) = log(1 + e^x), evaluated as max(x, 0) + log1p(e^{-|x|})
//   gate(x)     = exp(-c * softplus(x))       in (0, 1] for c > 0
//   sigmoid(x)  = 1 / (1 + e^{-x})
__device__ __forceinline__ float softplus_f(float x) { return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))); }
__device__ __forceinline__ float gate_map(float x, float c) { return expf(-c * softplus_f(x)); }
__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + expf(-x)); }

}  // namespace kda
