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

// Level tables a quantized weight can use (the choice is not stored with it;
// every call on the weight passes the same one).
constexpr int kTableNf4 = 0;      // the NF4 table above
constexpr int kTableUniform = 1;  // 16 equally spaced levels -1 + 2i/15
const Nf4Table& level_table(int table);

// Element formats of the fp weight handed to the quantization kernel.
constexpr int kWeightF32 = 0;
constexpr int kWeightBf16 = 1;
constexpr int kWeightF16 = 2;

// Decision tables of the quantization kernel (built on the host from the
// thresholds above, passed by value).  A normalized value y is first
// estimated as y' = x * rcp(s), within a few ulp of fl32(x / s).  The top 16
// bits of y' select a bucket: index 0 holds |y'| < 2^-6, index i >= 1 the
// bf16 interval starting at bits 0x3C7F + i; the sign picks one of two rows.
// Every bucket, widened by a relative 2^-19 on both sides, contains at most one
// threshold; kidx is the number of thresholds below it, so the level index is
// kidx + [fl32(x / s) > thr[kidx]], and that one comparison is made exactly
// as x > s * mid[kidx] in double precision (mid[k] is the midpoint between
// thr[k] and the next float32 above it; s * mid is exact in double, and
// x / s never equals mid, so no tie can occur).  mid[15] = +inf.
constexpr int kLutSide = 770;
struct QuantLut {
  uint8_t kidx[2 * kLutSide + 4];  // [sign][bucket], padded to whole words
  double mid[16];
};

// The table above (NF4, or that of level table `table`); ok is false if some
// widened bucket held two thresholds.
const QuantLut& quant_lut(int table, bool* ok);

// Workgroup barrier that orders LDS only: waits for this wave's LDS
// operations, then s_barrier.  (__syncthreads() also waits for every
// outstanding global load, which would drain loads issued ahead.)  The asm is
// a compiler memory barrier, so no LDS access moves across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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
// The quotient is formed without a division: q = c_g * fl32(1/255) is within
// an ulp, and one residual step r = c_g - 255 q (exact in an FMA),
// q + r * fl32(1/255) rounds to the correctly rounded quotient for every
// finite c_g >= 0 (checked over all such floats).  c_g = inf or NaN leaves r
// NaN; q is then the IEEE quotient itself.
__device__ __forceinline__ float scale_step(float c_g) {
  constexpr float inv = 1.0f / 255.0f;
  const float q = c_g * inv;
  const float r = __builtin_fmaf(-q, 255.0f, c_g);
  return r == r ? __builtin_fmaf(r, inv, q) : q;
}
__device__ __forceinline__ float restored_scale(uint32_t code, float c_g) {
  return (float)code * scale_step(c_g);
}

}  // namespace qlora
