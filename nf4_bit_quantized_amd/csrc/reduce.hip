// Fixed-order reductions of split-contraction partials and small elementwise
// steps of the rank-r adapter products (no atomics: results are deterministic).
#include "common.hpp"
#include "trace.hpp"

namespace qlora {

// V[t][j] = sum_z P[z][t][j] (j < r).  Writes V (fp32, may be NULL) and the
// bf16 hi/lo pair of s*V into Hs[t][0..r) and Hs[t][r..2r); Hs columns
// [2r, ldh) are zeroed.  With nsplit == 1 and P = an fp32 [T][r] tensor this
// only forms the hi/lo pair.
__global__ __launch_bounds__(256) void k_reduce_lowrank(const float* __restrict__ P, int nsplit,
                                                        int64_t split_stride, int64_t T, int r,
                                                        float s, float* __restrict__ V,
                                                        uint16_t* __restrict__ Hs, int64_t ldh) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= T * ldh) return;
  const int64_t t = idx / ldh;
  const int c = (int)(idx - t * ldh);
  if (c < r) {
    float v = 0.0f;
    for (int z = 0; z < nsplit; ++z) v += P[(int64_t)z * split_stride + t * r + c];
    if (V) V[t * r + c] = v;
    uint16_t hi, lo;
    split_bf16(s * v, hi, lo);
    Hs[t * ldh + c] = hi;
    Hs[t * ldh + r + c] = lo;
  } else if (c >= 2 * r) {
    Hs[t * ldh + c] = 0;
  }
}

// out[m][c] = sum_z (P[z][m][c] + P[z][m][c + r]), c < r; P rows have 2r columns.
__global__ __launch_bounds__(256) void k_reduce_colpairs(const float* __restrict__ P, int nsplit,
                                                         int64_t split_stride, int64_t M, int r,
                                                         float* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * r) return;
  const int64_t m = idx / r;
  const int c = (int)(idx - m * r);
  float v = 0.0f;
  for (int z = 0; z < nsplit; ++z) {
    const float* pz = P + (int64_t)z * split_stride + m * 2 * r;
    v += pz[c] + pz[c + r];
  }
  out[idx] = v;
}

// out[j][k] = sum_z (P[z][j][k] + P[z][j + r][k]), j < r; P has 2r rows of K.
__global__ __launch_bounds__(256) void k_reduce_rowpairs(const float* __restrict__ P, int nsplit,
                                                         int64_t split_stride, int r, int64_t K,
                                                         float* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)r * K) return;
  float v = 0.0f;
  for (int z = 0; z < nsplit; ++z) {
    const float* pz = P + (int64_t)z * split_stride;
    v += pz[idx] + pz[idx + (int64_t)r * K];
  }
  out[idx] = v;
}

__global__ __launch_bounds__(256) void k_fill_zero_f32(float* __restrict__ p, int64_t n) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx < n) p[idx] = 0.0f;
}

static unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

hipError_t launch_reduce_lowrank(const float* P, int nsplit, int64_t split_stride, int64_t T, int r,
                                 float s, float* V, uint16_t* Hs, int64_t ldh, hipStream_t stream) {
  if (T * ldh == 0) return hipSuccess;
  TraceScope ts(KID_REDUCE, stream);
  hipLaunchKernelGGL(k_reduce_lowrank, dim3(blocks_for(T * ldh)), dim3(256), 0, stream, P, nsplit,
                     split_stride, T, r, s, V, Hs, ldh);
  return hipGetLastError();
}

hipError_t launch_reduce_colpairs(const float* P, int nsplit, int64_t split_stride, int64_t M, int r,
                                  float* out, hipStream_t stream) {
  if (M * r == 0) return hipSuccess;
  TraceScope ts(KID_REDUCE, stream);
  hipLaunchKernelGGL(k_reduce_colpairs, dim3(blocks_for(M * r)), dim3(256), 0, stream, P, nsplit,
                     split_stride, M, r, out);
  return hipGetLastError();
}

hipError_t launch_reduce_rowpairs(const float* P, int nsplit, int64_t split_stride, int r, int64_t K,
                                  float* out, hipStream_t stream) {
  if ((int64_t)r * K == 0) return hipSuccess;
  TraceScope ts(KID_REDUCE, stream);
  hipLaunchKernelGGL(k_reduce_rowpairs, dim3(blocks_for((int64_t)r * K)), dim3(256), 0, stream, P,
                     nsplit, split_stride, r, K, out);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  TraceScope ts(KID_FILL, stream);
  hipLaunchKernelGGL(k_fill_zero_f32, dim3(blocks_for(n)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace qlora
