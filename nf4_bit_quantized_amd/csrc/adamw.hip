// AdamW update of the adapter parameters, with their bf16 copies for the next
// forward.
//
// "QLoRA技术从入门到精通" §3(3): after the backward pass the optimizer (an
// AdamW variant) updates only the adapter matrices A and B; the quantized base
// weight is never touched.  The arithmetic is the published AdamW method
// (Loshchilov and Hutter, "Decoupled Weight Decay Regularization"): decay on
// the parameter scaled by the learning rate, then the bias-corrected moment
// step.  Per element, in fp32, with the step-dependent factors formed on the
// host in double:
//
//   g  = grad * grad_scale
//   p  = p * (1 - lr * wd)
//   m  = beta1 * m + (1 - beta1) * g
//   v  = beta2 * v + (1 - beta2) * g * g
//   p  = p - (lr / (1 - beta1^t)) * m / (sqrt(v) / sqrt(1 - beta2^t) + eps)
//   p16 = bf16_rne(p)                                (optional)
//
// The parameters, gradients and both moments are flat fp32 arrays, so one
// launch can update every adapter of a model whose buffers are laid out in
// one arena.  HBM-bound: 16 bytes read and 12 (+2) written per element.
// Each thread takes two runs of four elements, all loads issued first; a
// ragged tail of fewer than four elements is done by one thread.
#pragma clang fp contract(off)

#include "adamw.hpp"
#include "trace.hpp"

namespace qlora {

namespace {

constexpr int kThreads = 256, kRuns = 2;

__device__ __forceinline__ void adamw_one(const AdamwParams& P, float& p, float g, float& m, float& v) {
  g = g * P.gscale;
  p = p * P.decay;
  m = P.beta1 * m + P.one_minus_beta1 * g;
  v = P.beta2 * v + P.one_minus_beta2 * (g * g);
  const float denom = sqrtf(v) * P.inv_sqrt_bc2 + P.eps;
  p = p - P.step_size * (m / denom);
}

__global__ __launch_bounds__(kThreads) void k_adamw(AdamwParams P) {
  typedef float f4_t __attribute__((ext_vector_type(4)));
  const int64_t n4 = P.n / 4;
  const int64_t base = (int64_t)blockIdx.x * kThreads * kRuns + threadIdx.x;
  f4_t p[kRuns], g[kRuns], m[kRuns], v[kRuns];
#pragma unroll
  for (int u = 0; u < kRuns; ++u) {
    const int64_t i = base + (int64_t)u * kThreads;
    if (i < n4) {
      p[u] = reinterpret_cast<const f4_t*>(P.p)[i];
      g[u] = reinterpret_cast<const f4_t*>(P.g)[i];
      m[u] = reinterpret_cast<const f4_t*>(P.m)[i];
      v[u] = reinterpret_cast<const f4_t*>(P.v)[i];
    }
  }
#pragma unroll
  for (int u = 0; u < kRuns; ++u) {
    const int64_t i = base + (int64_t)u * kThreads;
    if (i >= n4) continue;
    float pe[4] = {p[u].x, p[u].y, p[u].z, p[u].w};
    float me[4] = {m[u].x, m[u].y, m[u].z, m[u].w};
    float ve[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
    const float ge[4] = {g[u].x, g[u].y, g[u].z, g[u].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) adamw_one(P, pe[e], ge[e], me[e], ve[e]);
    reinterpret_cast<f4_t*>(P.p)[i] = f4_t{pe[0], pe[1], pe[2], pe[3]};
    reinterpret_cast<f4_t*>(P.m)[i] = f4_t{me[0], me[1], me[2], me[3]};
    reinterpret_cast<f4_t*>(P.v)[i] = f4_t{ve[0], ve[1], ve[2], ve[3]};
    if (P.p16) reinterpret_cast<uint2*>(P.p16)[i] = make_uint2(pack_bf16x2(pe[0], pe[1]), pack_bf16x2(pe[2], pe[3]));
  }
  // the ragged tail (n % 4 elements), by the grid's first thread
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    for (int64_t j = n4 * 4; j < P.n; ++j) {
      float pj = P.p[j], mj = P.m[j], vj = P.v[j];
      adamw_one(P, pj, P.g[j], mj, vj);
      P.p[j] = pj;
      P.m[j] = mj;
      P.v[j] = vj;
      if (P.p16) P.p16[j] = (uint16_t)(pack_bf16x2(pj, 0.0f) & 0xFFFFu);
    }
  }
}

}  // namespace

hipError_t launch_adamw(const AdamwParams& P, hipStream_t stream) {
  if (P.n <= 0) return hipSuccess;
  const int64_t n4 = P.n / 4;
  const int64_t per = (int64_t)kThreads * kRuns;
  const int64_t blocks = n4 > 0 ? (n4 + per - 1) / per : 1;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  KernelEvents ev(KID_ADAMW);
  hipExtLaunchKernelGGL(k_adamw, dim3((unsigned)blocks), dim3(kThreads), 0, stream, ev.start(), ev.stop(), 0, P);
  return hipGetLastError();
}

}  // namespace qlora
