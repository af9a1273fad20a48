// Parameters of the streaming rank-r adapter products (see lora_stream.hip).
#pragma once

#include "common.hpp"

namespace qlora {

// C[m][j] = sum_{c < D} P[m][c] Qop[j][c], m < M, j < r, then the hi/lo pair of
// s*C into Hout (zero-padded to ldh) and, optionally, C itself into Vout.
struct RowsParams {
  const uint16_t* P;  // bf16 [M][ldp], 16-byte aligned, ldp % 8 == 0
  int64_t ldp;
  int64_t M, D;       // rows; contraction length (a multiple of 64)
  const uint16_t* Q;  // q_strided == 0: Qop[j][c] = Q[j*ldq + c]; 1: Q[c*r + j] ([D][r], ldq == r)
  int64_t ldq;
  int32_t q_strided;
  int32_t r;          // a multiple of 8, at most 64
  float s;
  float* Vout;        // optional fp32 [M][r]
  uint16_t* Hout;     // bf16 [M][ldh]
  int64_t ldh;
  // optional: Ucs[m][..] = hi/lo pair of s * Uc[m][0..r) for the same rows, zero-padded to ldh
  const float* Uc;
  uint16_t* Ucs;
};

// Fout = sum_t P[t][m] (Q[t][j] + Q[t][j + r]), m < D, j < r: Fout[m][j], or
// Fout[j][m] when transposed_out.
struct ColsParams {
  const uint16_t* P;  // bf16 [T][ldp], 16-byte aligned, ldp % 8 == 0
  int64_t ldp;
  int64_t D;          // a multiple of 8
  const uint16_t* Q;  // bf16 [T][ldq] (hi columns 0..r-1, lo columns r..2r-1), 16-byte aligned
  int64_t ldq;
  int64_t T;
  int32_t r;          // a multiple of 8, at most 64 (the same for both products of a batch)
  int32_t transposed_out;
  float* Fout;
  int32_t accumulate;  // 1: Fout += result (gradient accumulation), 0: Fout = result
};

struct ColsBatch {
  ColsParams p[2];
  int n;
};

// U = X A^T for at most 16 tokens, in one launch: U [T][r] fp32 (optional),
// Us [T][ldh] the hi/lo pair of s*U, zero-padded.  X [T][K], A [r][K] bf16,
// 16-byte aligned, K a multiple of 8.
struct SmallDownParams {
  const uint16_t* X;
  const uint16_t* A;
  int64_t T, K;
  int32_t r;
  float s;
  float* U;
  uint16_t* Us;
  int64_t ldh;
};

bool lora_down_small_ok(int64_t T, int64_t K, int r);
hipError_t launch_lora_down_small(const SmallDownParams& p, hipStream_t stream, int kernel_id);

bool lora_stream_ok(int r);
bool lora_rows_ok(int64_t M, int r);
// part is workspace for the partial sums of the contraction ranges,
// lora_rows_part_bytes(M, D, r) bytes (0: none needed).
size_t lora_rows_part_bytes(int64_t M, int64_t D, int r);
hipError_t launch_lora_rows(const RowsParams& p, float* part, size_t part_bytes, hipStream_t stream, int kernel_id);
// dA and dB: part is workspace for the partial sums of the token ranges,
// lora_cols_part_bytes(T, {D of each product}, n, r) bytes (0: none needed).
size_t lora_cols_part_bytes(int64_t T, const int64_t* D, int n, int r);
hipError_t launch_lora_cols(const ColsBatch& B, float* part, size_t part_bytes, hipStream_t stream, int kernel_id);

}  // namespace qlora
