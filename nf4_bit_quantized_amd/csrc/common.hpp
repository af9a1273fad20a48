// Shared device-side types and helpers of the QLoRA NF4 library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

namespace qlora {

// The NF4 level table and the 15 decision thresholds, passed to kernels by
// value (kernel-argument memory).  Built on the host by nf4_table.cpp.
struct Nf4Table {
  float level[16];
  float thr[15];
};

const Nf4Table& nf4_table();

// Two fp32 -> packed bf16x2 (round to nearest even; low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t v = {a, b};
  bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float a) {
  return (uint16_t)(pack_bf16x2(a, 0.0f) & 0xFFFFu);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __builtin_bit_cast(float, h << 16);
}

// Split v into hi + lo with hi = bf16(v), lo = bf16(v - hi): the pair carries
// about 16 significant bits, enough to feed an fp32 value to a bf16 MFMA.
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16_bits(v);
  lo = f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
}

// Restored scale of a 64-weight block: fl32(fl32(code) * fl32(c_g / 255)).
__device__ __forceinline__ float restored_scale(uint32_t code, float c_g) {
  const float step = c_g / 255.0f;  // IEEE-rounded division
  return (float)code * step;
}

}  // namespace qlora
