// Host-visible description of the tiled bf16 MFMA contraction used by every
// dense step of the layer (forward base GEMM with fused LoRA term, dX with
// transposed dequant, the skinny adapter products U, G, dA, dB).
#pragma once

#include "common.hpp"

namespace qlora {

// How a logical operand Op[row][kk] (row = output row or column, kk = the
// contraction index) is read from memory.  Everything outside
// [0, rows) x [0, kdim) reads as zero.
enum OpKind : int {
  OP_ZERO = 0,
  OP_BF16_K = 1,  // Op[row][kk] = p[row * ld + src(kk)]           (contraction index contiguous)
  OP_BF16_T = 2,  // Op[row][kk] = p[src(kk) * ld + row]           (row index contiguous)
  OP_NF4_K = 3,   // Op[row=n][kk=k] = W_hat[n][k]                  (forward: restore along k)
  OP_NF4_T = 4,   // Op[row=k][kk=n] = W_hat[n][k]                  (dX: restore, transpose)
};

struct Operand {
  int32_t kind;
  int32_t kk_mod;        // bf16 kinds: src(kk) = kk % kk_mod (0: src(kk) = kk)
  const void* p;         // bf16 bits, or packed nibbles [N][K/2]
  const uint8_t* codes;  // NF4: 8-bit block scale codes [N*K/64]
  const float* consts;   // NF4: group constants
  int64_t ld;            // bf16: row stride in elements; NF4: K (d_in) of the stored weight
  int64_t rows;
  int64_t kdim;
};

struct Segment {
  Operand a, b;
  int64_t ktiles;  // ceil(kdim / 64)
};

enum OutKind : int {
  OUT_BF16 = 0,  // C -> bf16 bits at out[m * ldo + n]
  OUT_F32 = 1,   // C -> fp32 at out[z * split_stride + m * ldo + n] (split z of the contraction)
};

struct GemmParams {
  Segment seg[2];
  int32_t nseg;
  int32_t out_kind;
  void* out;
  int64_t ldo;
  int64_t split_stride;
  int64_t M, N;
  int32_t nsplit;
  int32_t tiles_per_split;
};

hipError_t launch_gemm(const GemmParams& p, hipStream_t stream, int kernel_id);

}  // namespace qlora
