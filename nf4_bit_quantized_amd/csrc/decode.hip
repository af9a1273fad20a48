// Forward for few tokens (T <= 16): stream the packed weight once.
//
// With at most 16 tokens the product X W_hat^T is bound by reading the
// packed nibbles and scale codes from HBM ("QLoRA技术从入门到精通" §3(2):
// the 4-bit weight is restored block by block at compute time and discarded).
// Each wave owns two 16-row strips of W and a slice of the contraction; every
// lane reads 16 packed bytes (32 consecutive weights of one row), restores
// them to bf16 in registers and feeds v_mfma_f32_16x16x32_bf16 with W as the
// 16 x 32 A operand and the tokens (zero-padded to 16) as the B operand,
// staged through LDS 512 columns at a time.  Partial sums over each
// contraction slice go to fp32 partials; k_decode_epilogue sums them in a
// fixed order, adds the rank-r term s * U B^T in fp32 and rounds to bf16.
//
// Lane <-> k mapping: MFMA j (0..3) of a 128-wide step uses, in lane l,
// weights k = step + 32*(l/16) + 8j + e for both operands, so the lane's 16
// packed bytes cover exactly the 32 weights it feeds.
#include "common.hpp"
#include "trace.hpp"

namespace qlora {

namespace {
constexpr int XCH = 512;         // k columns of X staged per LDS fill
constexpr int XLD = XCH + 8;     // padded LDS row (bf16 elements)
constexpr int ROWS_PER_WG = 128; // 4 waves x 2 strips x 16 rows
}  // namespace

__global__ __launch_bounds__(256) void k_decode_partial(const uint8_t* __restrict__ packed,
                                                        const uint8_t* __restrict__ codes,
                                                        const float* __restrict__ consts,
                                                        const uint16_t* __restrict__ X, int64_t T,
                                                        int64_t N, int64_t K, int64_t kchunk,
                                                        float* __restrict__ Ppart, Nf4Table tab) {
  __shared__ __attribute__((aligned(16))) uint16_t Xs[16 * XLD];
  __shared__ float lut[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t z = blockIdx.y;
  const int64_t kbeg = z * kchunk;
  const int64_t kend = kbeg + kchunk < K ? kbeg + kchunk : K;
  const int64_t nbase = (int64_t)blockIdx.x * ROWS_PER_WG + wave * 32;
  const bool wave_active = nbase < N;  // N is a multiple of 64: strips are all-in or all-out
  if (tid < 16) lut[tid] = tab.level[tid];

  f32x4_t acc[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) acc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t kb_row = K / 64;
  for (int64_t kx = kbeg; kx < kend; kx += XCH) {
    __syncthreads();
    for (int c = tid; c < 16 * (XCH / 8); c += 256) {
      const int t = c / (XCH / 8), kc = (c % (XCH / 8)) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (t < T && kx + kc < kend) v = *reinterpret_cast<const uint4*>(X + t * K + kx + kc);
      *reinterpret_cast<uint4*>(Xs + t * XLD + kc) = v;
    }
    __syncthreads();
    if (!wave_active) continue;
    const int64_t klen = kend - kx < XCH ? kend - kx : XCH;
    for (int ks = 0; ks < klen; ks += 128) {
      const int kl = ks + 32 * (lane >> 4);  // this lane's first k inside the staged chunk
      bf16x8_t xf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xf[j] = *reinterpret_cast<const bf16x8_t*>(Xs + (lane & 15) * XLD + kl + 8 * j);
      const bool kvalid = kl < klen;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int64_t n = nbase + s * 16 + (lane & 15);
        const int64_t k = kx + kl;
        uint32_t wv[4] = {0u, 0u, 0u, 0u};
        float sc = 0.0f;
        if (kvalid) {
          const uint4 pv = *reinterpret_cast<const uint4*>(packed + n * (K / 2) + k / 2);
          wv[0] = pv.x; wv[1] = pv.y; wv[2] = pv.z; wv[3] = pv.w;
          const int64_t blk = n * kb_row + k / 64;
          sc = restored_scale(codes[blk], consts[blk >> 8]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w = wv[j];
          uint32_t h[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const uint32_t byte = (w >> (8 * b)) & 0xFFu;
            h[b] = pack_bf16x2(lut[byte >> 4] * sc, lut[byte & 15u] * sc);
          }
          typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
          const u32x4_t hv = {h[0], h[1], h[2], h[3]};
          const bf16x8_t wf = __builtin_bit_cast(bf16x8_t, hv);
          acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, xf[j], acc[s], 0, 0, 0);
        }
      }
    }
  }
  if (!wave_active) return;
  // C[n][t]: lane holds token (lane & 15) and rows 4*(lane/16) + i of each strip
  const int t = lane & 15;
  if (t < T) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t n = nbase + s * 16 + 4 * (lane >> 4) + i;
        Ppart[z * T * N + t * N + n] = acc[s][i];
      }
  }
}

// Y[t][n] = bf16( sum_z P[z][t][n] + s * sum_j U[t][j] B[n][j] )
__global__ __launch_bounds__(256) void k_decode_epilogue(const float* __restrict__ Ppart, int nsplit,
                                                         int64_t T, int64_t N,
                                                         const float* __restrict__ U, int r, float s,
                                                         const uint16_t* __restrict__ B,
                                                         uint16_t* __restrict__ Y) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= T * N) return;
  const int64_t t = idx / N, n = idx - t * N;
  float acc = 0.0f;
  for (int z = 0; z < nsplit; ++z) acc += Ppart[(int64_t)z * T * N + idx];
  float lora = 0.0f;
  for (int j = 0; j < r; ++j) lora = fmaf(U[t * r + j], bf16_bits_to_f32(B[n * r + j]), lora);
  Y[idx] = f32_to_bf16_bits(acc + s * lora);
}

hipError_t launch_decode(const uint8_t* packed, const uint8_t* codes, const float* consts,
                         const uint16_t* X, int64_t T, int64_t N, int64_t K, int64_t kchunk,
                         int nsplit, float* Ppart, const float* U, int r, float s,
                         const uint16_t* B, uint16_t* Y, hipStream_t stream) {
  const dim3 grid((unsigned)((N + ROWS_PER_WG - 1) / ROWS_PER_WG), (unsigned)nsplit);
  {
    TraceScope ts(KID_DECODE, stream);
    hipLaunchKernelGGL(k_decode_partial, grid, dim3(256), 0, stream, packed, codes, consts, X, T, N, K,
                       kchunk, Ppart, nf4_table());
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = T * N;
  TraceScope ts(KID_DECODE_EPILOGUE, stream);
  hipLaunchKernelGGL(k_decode_epilogue, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     Ppart, nsplit, T, N, U, r, s, B, Y);
  return hipGetLastError();
}

}  // namespace qlora
