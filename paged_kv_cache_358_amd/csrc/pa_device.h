// Device-side helpers shared by the gfx950 kernels of the paged KV-cache library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedattn.h"

namespace pa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

constexpr int kWave = 64;
constexpr int kBlockTokens = 16;  // tokens per KV block handled by the kernels
constexpr float kLog2e = 1.4426950408889634f;

inline int elem_bytes(int32_t dtype) { return dtype == PA_F32 ? 4 : 2; }
inline bool valid_dtype(int32_t dtype) { return dtype == PA_F32 || dtype == PA_BF16 || dtype == PA_F16; }

// Element conversions (storage type <-> float).
__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float f16_bits_to_float(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}
// float -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t float_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

template <int DT> struct Elem;
template <> struct Elem<PA_F32> {
  using storage = float;
  __device__ static float to_float(float x) { return x; }
  __device__ static float from_float(float x) { return x; }
};
template <> struct Elem<PA_BF16> {
  using storage = uint16_t;
  __device__ static float to_float(uint16_t x) { return bf16_bits_to_float(x); }
  __device__ static uint16_t from_float(float x) { return static_cast<uint16_t>(float_to_bf16_bits(x)); }
};
template <> struct Elem<PA_F16> {
  using storage = uint16_t;
  __device__ static float to_float(uint16_t x) { return f16_bits_to_float(x); }
  __device__ static uint16_t from_float(float x) { return static_cast<uint16_t>(float_to_f16_bits(x)); }
};

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace pa
