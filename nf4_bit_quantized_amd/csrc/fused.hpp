// Parameters of the fused NF4-restore GEMMs (forward base product and dX).
#pragma once

#include "common.hpp"

namespace qlora {

// forward: C[M=T][N=d_out] = A(X)[T][K0=d_in] . W_hat^T + tail
// dX:      C[M=T][N=d_in]  = A(dY)[T][K0=d_out] . W_hat  + tail
struct FusedParams {
  const uint16_t* A;       // bf16 [M][lda], contraction contiguous
  int64_t lda;
  const uint8_t* packed;   // stored weight [d_out][d_in/2]
  const uint8_t* codes;
  const float* consts;
  int64_t Kw;              // d_in of the stored weight
  int64_t M, N, K0;        // output rows, output columns, main contraction length
  const uint16_t* At;      // tail A: bf16 [M][ldat] = hi/lo pair of s*U or s*G (2r columns used)
  int64_t ldat;
  const uint16_t* Bt;      // tail B source: B [d_out][r] (forward) or A [r][d_in] (dX)
  int64_t ldbt;
  int32_t r;               // rank (0: no tail)
  uint16_t* C;             // bf16 output [M][ldc]
  int64_t ldc;
  int32_t table;           // level table (kTableNf4 / kTableUniform)
  int32_t bshift;          // log2(weights per absmax block / 64)
  int32_t dq;              // 1: 8-bit codes + group constants; 0: consts holds the fp32 block scales
  int32_t accumulate;      // 1: C = bf16(C + tile), adding to what C holds (C's tile is rounded first)
  int32_t mt, nt, group_m; // filled by the launcher
  Nf4Table tab;            // filled by the launcher from table
};

hipError_t launch_fused(FusedParams P, bool dx, hipStream_t stream, int kernel_id);

}  // namespace qlora
