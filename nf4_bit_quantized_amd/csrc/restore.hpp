// Restore of NF4-packed weights to bf16 through per-block byte tables in
// registers, shared by the fused products and the export kernel.
//
// A thread that restores weights of one 64-weight block first builds the 16
// values bf16(T[i] * s') of that block (16 fp32 products, 8 pack-converts),
// split into a high-byte table and a low-byte table of four registers each;
// each 4-bit index is then resolved with v_perm_b32 byte selects (three per
// byte table per four indices), so a packed word of 8 indices costs 25 VALU
// instructions (selectors 9, lookups 12, pairing 4) and no memory access.  The
// values are exactly bf16_rne(fl32(T[q] * s')).
#pragma once

#include "common.hpp"

namespace qlora {

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// High-byte and low-byte tables of the 16 restored values of one block.
struct RestoreTab {
  uint32_t h[4], l[4];
};

__device__ __forceinline__ RestoreTab make_tab(const Nf4Table& tab, float sc) {
  uint32_t w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = pack_bf16x2(tab.level[2 * j] * sc, tab.level[2 * j + 1] * sc);
  RestoreTab t;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t.h[i] = perm(w[2 * i + 1], w[2 * i], 0x07050301u);
    t.l[i] = perm(w[2 * i + 1], w[2 * i], 0x06040200u);
  }
  return t;
}

// Byte selectors of four 4-bit indices: sl picks, in each byte, the index's
// entry inside the low (0-7) or high (8-15) half of a table (its low three
// bits), s2 then picks per byte between the two halves' results (bit 3).
// Even elements are the high nibbles of the packed word, odd ones the low
// nibbles; the selectors are formed straight from the word.
// (x & 0x04040404) | 0x03020100 as one v_and_or_b32: its two constants are
// held in vector registers, since a VOP3 instruction takes neither two scalar
// operands nor a literal here.
__device__ __forceinline__ uint32_t half_select(uint32_t x) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(0x04040404u), "v"(0x03020100u));
  return r;
}
__device__ __forceinline__ void selectors_even(uint32_t w, uint32_t& sl, uint32_t& s2) {
  sl = (w >> 4) & 0x07070707u;
  s2 = half_select(w >> 5);
}
__device__ __forceinline__ void selectors_odd(uint32_t w, uint32_t& sl, uint32_t& s2) {
  sl = w & 0x07070707u;
  s2 = half_select(w >> 1);
}

// The high and low bytes of the four restored values the selectors name, one per byte.
__device__ __forceinline__ void lookup4(uint32_t sl, uint32_t s2, const RestoreTab& t, uint32_t& H, uint32_t& L) {
  H = perm(perm(t.h[3], t.h[2], sl), perm(t.h[1], t.h[0], sl), s2);
  L = perm(perm(t.l[3], t.l[2], sl), perm(t.l[1], t.l[0], sl), s2);
}

// Four consecutive indices of a packed word, one per byte (in the low nibble;
// the high nibble is ignored by the selectors): q = 0 gathers elements 0-3,
// q = 1 elements 4-7.  Element 2j is the high nibble of byte j, so it is the
// low nibble of byte j of w >> 4 (w4), and element 2j+1 that of byte j of w.
__device__ __forceinline__ uint32_t gather4(uint32_t w, uint32_t w4, int q) {
  return perm(w4, w, q == 0 ? 0x01050004u : 0x03070206u);
}
__device__ __forceinline__ void selectors(uint32_t x, uint32_t& sl, uint32_t& s2) {
  sl = x & 0x07070707u;
  s2 = half_select(x >> 1);
}

// One packed word (8 indices, element 2j in the high nibble of byte j) ->
// four words of bf16 pairs in element order.  The selectors take the indices
// in element order, so each lookup's high and low bytes pair up directly.
__device__ __forceinline__ void restore8(uint32_t w, const RestoreTab& t, uint32_t* out) {
  const uint32_t w4 = w >> 4;
  uint32_t sl, s2, H, L;
  selectors(gather4(w, w4, 0), sl, s2);
  lookup4(sl, s2, t, H, L);
  out[0] = perm(H, L, 0x05010400u);
  out[1] = perm(H, L, 0x07030602u);
  selectors(gather4(w, w4, 1), sl, s2);
  lookup4(sl, s2, t, H, L);
  out[2] = perm(H, L, 0x05010400u);
  out[3] = perm(H, L, 0x07030602u);
}

// A restore whose selectors come straight from the word's nibble planes (no
// gather): the words hold the bf16 pairs (e0, e2), (e4, e6), (e1, e3),
// (e5, e7) -- elements in the order 0, 2, 4, 6, 1, 3, 5, 7.  A product that
// takes its operand in this order on both sides (or undoes it on its output)
// saves two instructions per word over restore8.
__device__ __forceinline__ void restore8_evenodd(uint32_t w, const RestoreTab& t, uint32_t* out) {
  uint32_t HE, LE, HO, LO, sl, s2;
  selectors_even(w, sl, s2);
  lookup4(sl, s2, t, HE, LE);
  selectors_odd(w, sl, s2);
  lookup4(sl, s2, t, HO, LO);
  out[0] = perm(HE, LE, 0x05010400u);
  out[1] = perm(HE, LE, 0x07030602u);
  out[2] = perm(HO, LO, 0x05010400u);
  out[3] = perm(HO, LO, 0x07030602u);
}

}  // namespace qlora
