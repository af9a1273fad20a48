// LoRA dropout on the adapter's input.
//
// "LoRA 与 QLoRA：把大模型微调拆成可负担的工程" §4.3: LoRA dropout randomly
// drops elements of the adapter's input (its §8 configuration: 0.05); the base
// branch keeps the whole input.  Inverted dropout in the 16-bit compute type:
//   X_d = bf16_rne(fl32(x * c)) where kept, 0 where dropped, c = fl32(1 / (1 - p)).
// The keep mask is an input: [T][K/8] bytes, bit j of byte i (least
// significant first) keeps element 8i + j.
//
// k_dropout_input writes X_d (the adapter's down product and dA read it).
// k_dropout_dx_add adds the adapter's share of dX, which the chain rule sends
// back through the same mask and factor, to the base share dY W_hat already
// in dX:
//   dX = bf16_rne( fl32(dX) + keep * c * sum_j sG[t][j] A[j][k] ),
// with s G given as its bf16 hi/lo pair (the form the rank-r tails use).
// Both are HBM-bound elementwise passes; the rank-r sum is fp32 FMAs on the
// vector ALUs (r per element), A's rows coming from L2.
#pragma clang fp contract(off)

#include "dropout.hpp"
#include "trace.hpp"

namespace qlora {

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// one thread: 8 consecutive elements (16 bytes of X, one mask byte)
__global__ __launch_bounds__(256) void k_dropout_input(const uint16_t* __restrict__ X, const uint8_t* __restrict__ keep,
                                                       float c, int64_t n8, uint16_t* __restrict__ Xd) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const u32x4_t x = reinterpret_cast<const u32x4_t*>(X)[i];
  const uint32_t m = keep[i];
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float a = (m >> (2 * q)) & 1u ? bf16lo(w[q]) * c : 0.0f;
    const float b = (m >> (2 * q + 1)) & 1u ? bf16hi(w[q]) * c : 0.0f;
    o[q] = pack_bf16x2(a, b);
  }
  reinterpret_cast<u32x4_t*>(Xd)[i] = u32x4_t{o[0], o[1], o[2], o[3]};
}

constexpr int DT = 4;      // token rows per workgroup
constexpr int DCOL = 8;    // columns per thread

// Workgroup: DT token rows x 256*8 columns.  s G of the rows goes to LDS as
// fp32 (hi + lo), transposed so that one read gives column j for all DT rows;
// each thread then walks j, loading its 8 columns of A row j (from L2).
__global__ __launch_bounds__(256) void k_dropout_dx_add(DropoutDxParams P) {
  extern __shared__ float sg[];  // [r][DT]
  const int64_t t0 = (int64_t)blockIdx.y * DT;
  const int64_t k0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * DCOL;
  const int rows = (int)((P.T - t0) < DT ? (P.T - t0) : DT);
  for (int e = threadIdx.x; e < P.r * DT; e += 256) {
    const int j = e / DT, t = e % DT;
    float v = 0.0f;
    if (t < rows) {
      const uint16_t* g = P.Gs + (t0 + t) * P.ldh;
      v = __builtin_bit_cast(float, (uint32_t)g[j] << 16) + __builtin_bit_cast(float, (uint32_t)g[P.r + j] << 16);
    }
    sg[j * DT + t] = v;
  }
  __syncthreads();
  if (k0 >= P.K) return;
  // the rows' dX pieces and mask bytes are loaded first, so their latency
  // hides under the rank-r sums
  u32x4_t d[DT];
  uint32_t m[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    const int64_t row = t0 + (t < rows ? t : 0);
    d[t] = *reinterpret_cast<const u32x4_t*>(P.dX + row * P.K + k0);
    m[t] = P.keep[row * (P.K / 8) + k0 / 8];
  }
  float acc[DT][DCOL];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int e = 0; e < DCOL; ++e) acc[t][e] = 0.0f;
  for (int j = 0; j < P.r; ++j) {
    const u32x4_t a4 = *reinterpret_cast<const u32x4_t*>(P.A + (int64_t)j * P.K + k0);
    const float a[DCOL] = {bf16lo(a4.x), bf16hi(a4.x), bf16lo(a4.y), bf16hi(a4.y),
                           bf16lo(a4.z), bf16hi(a4.z), bf16lo(a4.w), bf16hi(a4.w)};
    float g[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) g[t] = sg[j * DT + t];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int e = 0; e < DCOL; ++e) acc[t][e] = fmaf(g[t], a[e], acc[t][e]);
  }
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    if (t >= rows) break;
    const uint32_t w[4] = {d[t].x, d[t].y, d[t].z, d[t].w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float l0 = (m[t] >> (2 * q)) & 1u ? P.c * acc[t][2 * q] : 0.0f;
      const float l1 = (m[t] >> (2 * q + 1)) & 1u ? P.c * acc[t][2 * q + 1] : 0.0f;
      o[q] = pack_bf16x2(bf16lo(w[q]) + l0, bf16hi(w[q]) + l1);
    }
    *reinterpret_cast<u32x4_t*>(P.dX + (t0 + t) * P.K + k0) = u32x4_t{o[0], o[1], o[2], o[3]};
  }
}

}  // namespace

hipError_t launch_dropout_input(const uint16_t* X, const uint8_t* keep, float c, int64_t T, int64_t K, uint16_t* Xd,
                                hipStream_t stream) {
  if (K % 8 != 0) return hipErrorInvalidValue;
  const int64_t n8 = T * K / 8;
  if (n8 == 0) return hipSuccess;
  KernelEvents ev(KID_DROPOUT);
  hipExtLaunchKernelGGL(k_dropout_input, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, ev.start(),
                        ev.stop(), 0, X, keep, c, n8, Xd);
  return hipGetLastError();
}

hipError_t launch_dropout_dx_add(const DropoutDxParams& P, hipStream_t stream) {
  if (P.K % DCOL != 0 || P.r < 1 || P.r > 128) return hipErrorInvalidValue;
  if (P.T == 0) return hipSuccess;
  const dim3 grid((unsigned)((P.K + 256 * DCOL - 1) / (256 * DCOL)), (unsigned)((P.T + DT - 1) / DT));
  KernelEvents ev(KID_DROPOUT);
  hipExtLaunchKernelGGL(k_dropout_dx_add, grid, dim3(256), (uint32_t)(P.r * DT * 4), stream, ev.start(), ev.stop(), 0,
                        P);
  return hipGetLastError();
}

}  // namespace qlora
