// Few-token forward (see decode.hip).
#pragma once

#include "common.hpp"

namespace qlora {

// One weight of a (possibly multi-weight) few-token forward.
struct DecodeWeight {
  const uint8_t* packed;
  const uint8_t* codes;
  const float* consts;
  int64_t N;           // rows
  const uint16_t* B;   // [N][r] bf16
  uint16_t* Y;         // [T][N] bf16
  int table;           // level table
};

constexpr int kDecodeMaxWeights = 4;

// f32s: fp32 block scales in consts (no second level, no codes)
bool decode_supported(int64_t N, int64_t K, int bshift, bool f32s);
// Workgroups per run of tiles that split the contraction (1 or 2; see decode.hip),
// and the bytes of their partial sums ([split][T][N] fp32; 0 without a split).
int decode_split(int64_t T, int64_t N, int64_t K, int bshift, bool f32s);
size_t decode_part_bytes(int64_t T, int64_t N, int64_t K, int bshift, bool f32s);
// part: decode_part_bytes(...) bytes of workspace; with fewer, the contraction is not split.
hipError_t launch_decode(const uint8_t* packed, const uint8_t* codes, const float* consts, const uint16_t* X,
                         int64_t T, int64_t N, int64_t K, const uint16_t* Us, int64_t ldh, const uint16_t* B,
                         int r, uint16_t* Y, int table, int bshift, bool f32s, float* part, size_t part_bytes,
                         hipStream_t stream);
// Up to kDecodeMaxWeights weights sharing X (and T, K, r, the block format) in
// one launch; Us[i] is weight i's hi/lo pair of s*U.
hipError_t launch_decode_multi(const DecodeWeight* w, int n, const uint16_t* X, int64_t T, int64_t K,
                               const uint16_t* const* Us, int64_t ldh, int r, int bshift, bool f32s,
                               hipStream_t stream);

}  // namespace qlora
