// Small elementwise kernels of the library.
#include "common.hpp"
#include "trace.hpp"

namespace qlora {

__global__ __launch_bounds__(256) void k_fill_zero_f32(float* __restrict__ p, int64_t n) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx < n) p[idx] = 0.0f;
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  TraceScope ts(KID_FILL, stream);
  hipLaunchKernelGGL(k_fill_zero_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace qlora
