// Parameters of the AdamW update of the adapter parameters (see adamw.hip).
#pragma once

#include "common.hpp"

namespace qlora {

struct AdamwParams {
  float* p;
  const float* g;
  float* m;
  float* v;
  uint16_t* p16;  // optional
  int64_t n;
  float decay;       // 1 - lr * wd
  float gscale;
  float beta1, one_minus_beta1, beta2, one_minus_beta2;
  float step_size;   // lr / (1 - beta1^t)
  float inv_sqrt_bc2;  // 1 / sqrt(1 - beta2^t)
  float eps;
};

hipError_t launch_adamw(const AdamwParams& P, hipStream_t stream);

}  // namespace qlora
