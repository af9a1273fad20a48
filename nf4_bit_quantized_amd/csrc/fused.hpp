// Parameters of the fused NF4-restore GEMMs (forward base product and dX).
#pragma once

#include "common.hpp"

namespace qlora {

constexpr int kMaxFusedSegs = 4;

// One further weight of a product over several weights (see FusedParams).
struct FusedSeg {
  const uint16_t* A;       // dX: this weight's dY [M][lda]; forward: unused (X is shared)
  int64_t lda;
  const uint8_t* packed;
  const uint8_t* codes;
  const float* consts;
  int64_t N;               // d_out of this weight
  const uint16_t* At;      // its hi/lo pair of s*U (forward) or s*G (dX)
  int64_t ldat;
  const uint16_t* Bt;      // its B (forward) or A (dX)
  int64_t ldbt;
  uint16_t* C;             // forward: its Y
  int64_t ldc;
};

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
  int64_t col0;            // dX on the 256 x 128 tiles: the weight column of output column 0 (C and the
                           // tail's Bt already point there); 0 otherwise
  int32_t mt, nt, group_m; // filled by the launcher
  Nf4Table tab;            // filled by the launcher from table
  // A product over several weights that share the activation (the projections
  // of one layer input): nseg > 1 and segments 1 .. nseg-1 below; segment 0
  // is the weight above.  Forward: the segments' output columns follow each
  // other (each weight's own Y); dX: their contraction rows follow each other
  // (each weight's own dY), all summed into one dX.
  int32_t nseg;
  FusedSeg seg[kMaxFusedSegs];
  int32_t seg_first[kMaxFusedSegs + 1];  // filled by the launcher: first tile column (forward) of each segment
};

hipError_t launch_fused(FusedParams P, bool dx, hipStream_t stream, int kernel_id);

// Choosing between the 256 x 256 kernels and the 256 x 128 one: `tiles`
// workgroups take ceil(tiles / 256) rounds of the GPU (one per CU), and a
// round of 256 x 256 tiles costs about 1.9 rounds of 256 x 128 ones (twice
// the work, done a few per cent faster per flop).  Costs in tenths of a
// 256 x 128 round.
inline int64_t gpu_rounds(int64_t tiles) { return (tiles + 255) / 256; }
inline int64_t wide_cost(int64_t tiles) { return 19 * gpu_rounds(tiles); }
inline int64_t narrow_cost(int64_t tiles) { return 10 * gpu_rounds(tiles); }

// The forward product on 256 x 256 tiles with the restore in the multiplying
// waves' registers (fused_wide.hip); launch_fused picks it where it applies.
bool fused_wide_ok(const FusedParams& P, bool dx);
hipError_t launch_fused_wide(FusedParams P, hipStream_t stream, int kernel_id);

// dX on 256 x 256 tiles with the restore done by the multiplying waves
// (fused_dx_wide.hip); launch_fused picks it where it applies.
bool fused_dx_wide_ok(const FusedParams& P);
hipError_t launch_fused_dx_wide(FusedParams P, hipStream_t stream, int kernel_id);

}  // namespace qlora
