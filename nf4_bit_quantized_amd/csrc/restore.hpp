// Restore of NF4-packed weights to bf16 through per-block byte tables in
// registers, shared by the fused products and the export kernel.
//
// A thread that restores weights of one 64-weight block first builds the 16
// values bf16(T[i] * s') of that block (16 fp32 products, 8 pack-converts),
// split into a high-byte table and a low-byte table of four registers each;
// each 4-bit index is then resolved with v_perm_b32 byte selects (three per
// byte table per four indices), so a packed word of 8 indices costs about 29
// VALU instructions and no memory access.  The values are exactly
// bf16_rne(fl32(T[q] * s')).
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

// n holds four 4-bit indices, one per byte; returns the high and low bytes of
// their restored bf16 values, one per byte.
__device__ __forceinline__ void lookup4(uint32_t n, const RestoreTab& t, uint32_t& H, uint32_t& L) {
  const uint32_t sl = n & 0x07070707u;
  const uint32_t s2 = ((n >> 1) & 0x04040404u) | 0x03020100u;
  H = perm(perm(t.h[3], t.h[2], sl), perm(t.h[1], t.h[0], sl), s2);
  L = perm(perm(t.l[3], t.l[2], sl), perm(t.l[1], t.l[0], sl), s2);
}

// One packed word (8 indices, element 2j in the high nibble of byte j) ->
// four words of bf16 pairs in element order.
__device__ __forceinline__ void restore8(uint32_t w, const RestoreTab& t, uint32_t* out) {
  uint32_t HE, LE, HO, LO;
  lookup4((w >> 4) & 0x0F0F0F0Fu, t, HE, LE);
  lookup4(w & 0x0F0F0F0Fu, t, HO, LO);
  const uint32_t e01 = perm(HE, LE, 0x05010400u), e23 = perm(HE, LE, 0x07030602u);
  const uint32_t o01 = perm(HO, LO, 0x05010400u), o23 = perm(HO, LO, 0x07030602u);
  out[0] = perm(o01, e01, 0x05040100u);
  out[1] = perm(o01, e01, 0x07060302u);
  out[2] = perm(o23, e23, 0x05040100u);
  out[3] = perm(o23, e23, 0x07060302u);
}

}  // namespace qlora
