// Parameters of the rank-r adapter products (see skinny.hip).
#pragma once

#include "common.hpp"

namespace qlora {

enum SkinnyQ : int {
  Q_CONTIG = 0,   // Qop[j][c] = Q[j*ldq + c]  (contraction contiguous)
  Q_STRIDED = 1,  // Qop[j][c] = Q[c*ldq + j]
  Q_HILO = 2,     // Qop[j][c] = hi/lo of s*V[c*ldv + j mod r]  (fp32 source)
};

enum SkinnyOut : int {
  OUT_ROWS_HILO = 0,  // C[m][j<r] -> Vout fp32 [mrows][r] (optional), Hout hi/lo bf16 [mrows][ldh]
  OUT_PAIRS = 1,      // Fout[m][j] = C[m][j] + C[m][j+r]      (fp32 [mrows][r])
  OUT_PAIRS_T = 2,    // Fout[j][m] = C[m][j] + C[m][j+r]      (fp32 [r][mrows])
  OUT_PARTIAL = 3,    // internal: fp32 partials [nsplit][mrows][ocols]
};

// C[m][j] = sum_{c < clen} Pop[m][c] Qop[j][c], m < mrows, j < qcols.
struct SkinnyParams {
  const uint16_t* P;  // bf16
  int64_t ldp;
  bool p_contig;      // Pop[m][c] = P[m*ldp + c]; otherwise P[c*ldp + m]
  bool pvec;          // 16-byte loads allowed
  const uint16_t* Q;  // bf16 (Q_CONTIG / Q_STRIDED)
  int64_t ldq;
  int64_t qrows;      // valid j rows of Q
  bool qvec;
  int32_t q_mode;
  const float* V;     // fp32 source for Q_HILO
  int64_t ldv;
  int32_t r;
  float s;
  int64_t mrows, clen;
  int32_t qcols;      // output columns (r or 2r)
  int32_t ocols;      // set by the launcher
  int32_t out_mode;
  int32_t nsplit;     // splits of the contraction over the grid
  float* Pout;        // partials (workspace) when nsplit > 1
  float* Vout;
  uint16_t* Hout;
  int64_t ldh;
  float* Fout;
  int32_t accumulate; // OUT_PAIRS / OUT_PAIRS_T: 1 adds the result to Fout, 0 overwrites it
  // optional (OUT_ROWS_HILO products of r columns): Ucs[m][..] = hi/lo pair
  // of s * Uc[m][0..r) for the same rows m, zero-padded to ldh
  const float* Uc;
  uint16_t* Ucs;
  int32_t sum_per_wg; // set by the launcher: outputs per workgroup of the split-partial sum
};

// Up to two independent products in one launch (blockIdx.z picks one).
struct SkinnyBatch {
  SkinnyParams p[2];
  int n;
};

int skinny_width(int cols);
int skinny_splits(int64_t mrows, int64_t clen, int cols);
hipError_t launch_skinny(SkinnyParams S, hipStream_t stream, int kernel_id);
// Two products with the same operand modes and width (P strided, Q strided).
hipError_t launch_skinny_pair(SkinnyParams S0, SkinnyParams S1, hipStream_t stream, int kernel_id);

}  // namespace qlora
