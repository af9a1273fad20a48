// Parameters of the LoRA-dropout kernels (see dropout.hip).
#pragma once

#include "common.hpp"

namespace qlora {

// dX[t][k] = bf16(dX[t][k] + keep[t][k] * c * sum_j sG[t][j] A[j][k])
struct DropoutDxParams {
  uint16_t* dX;           // bf16 [T][K], holds dY W_hat on entry
  const uint16_t* Gs;     // hi/lo bf16 pair of s*G, [T][ldh] (hi columns 0..r-1, lo r..2r-1)
  int64_t ldh;
  const uint16_t* A;      // bf16 [r][K], 16-byte aligned
  const uint8_t* keep;    // [T][K/8] keep bits
  float c;                // fl32(1 / (1 - p))
  int64_t T, K;
  int r;
};

hipError_t launch_dropout_input(const uint16_t* X, const uint8_t* keep, float c, int64_t T, int64_t K, uint16_t* Xd,
                                hipStream_t stream);
hipError_t launch_dropout_dx_add(const DropoutDxParams& P, hipStream_t stream);

}  // namespace qlora
