// Offline NF4 quantization of the base weight with double-quantized scales.
//
// "QLoRA技术从入门到精通" §3(1): the weight is cut into blocks of 64
// consecutive values; each block keeps its absmax as scale; values are
// divided by the scale into [-1, 1]; each is replaced by the index of the
// nearest NF4 level (4 bits, two per byte); the fp32 block scales are then
// gathered and quantized again to 8 bits.  Second-level format (the pages do
// not fix it): groups of 256 consecutive scales, one fp32 constant per group
// (its largest scale), unsigned 8-bit codes linear on [0, c_g] rounded half
// to even.  Indices use the exact block scale.
//
// One workgroup = one second-level group = 256 blocks = 16384 weights.
// 256 threads; thread t loads float4 number i*256 + t (i = 0..15) of the
// group, so each load instruction is a fully coalesced 4 KiB row; a float4
// belongs to block i*16 + t/16, shared by 16 consecutive lanes, whose absmax
// is reduced with four xor-shuffles inside those 16 lanes.  Results are
// bit-exact: IEEE division for x = w / s and for s / c_g, comparisons against
// exact thresholds, rint for the codes.  No floating-point contraction.
#pragma clang fp contract(off)

#include "common.hpp"
#include "trace.hpp"

namespace qlora {

__global__ __launch_bounds__(256) void k_nf4_quantize(const float* __restrict__ W,
                                                      uint8_t* __restrict__ packed,
                                                      uint8_t* __restrict__ codes,
                                                      float* __restrict__ consts, int64_t nb,
                                                      Nf4Table tab) {
  __shared__ float sh_scale[256];
  __shared__ float sh_wmax[4];

  const int t = threadIdx.x;
  const int64_t g = blockIdx.x;
  const int64_t blk0 = g * 256;
  const int nblk = (int)((nb - blk0) < 256 ? (nb - blk0) : 256);
  typedef float f4_t __attribute__((ext_vector_type(4)));
  const f4_t* src = reinterpret_cast<const f4_t*>(W) + blk0 * 16;

  f4_t v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int b = i * 16 + (t >> 4);
    if (b < nblk) {
      v[i] = __builtin_nontemporal_load(src + i * 256 + t);
    } else {
      v[i] = f4_t{0.f, 0.f, 0.f, 0.f};
    }
  }

  // absmax of each block: 4 values per lane, then 16 lanes
  float s[16];
  float tmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float m = fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w)));
    m = fmaxf(m, __shfl_xor(m, 8, 16));
    m = fmaxf(m, __shfl_xor(m, 4, 16));
    m = fmaxf(m, __shfl_xor(m, 2, 16));
    m = fmaxf(m, __shfl_xor(m, 1, 16));
    s[i] = m;
    tmax = fmaxf(tmax, m);
    if ((t & 15) == 0) sh_scale[i * 16 + (t >> 4)] = m;
  }

  // group constant c_g = max block scale (all 256 blocks of the group)
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
  if ((t & 63) == 0) sh_wmax[t >> 6] = tmax;
  __syncthreads();
  const float cg = fmaxf(fmaxf(sh_wmax[0], sh_wmax[1]), fmaxf(sh_wmax[2], sh_wmax[3]));

  if (t < nblk) {
    uint32_t code = 0;
    if (cg > 0.0f) {
      const float ratio = sh_scale[t] / cg;
      const float scaled = ratio * 255.0f;
      float r = rintf(scaled);
      r = fminf(fmaxf(r, 0.0f), 255.0f);
      code = (uint32_t)r;
    }
    codes[blk0 + t] = (uint8_t)code;
  }
  if (t == 0) consts[g] = cg;

  // indices: x = w / s, q = #{k : x > thr[k]}; two nibbles per byte, element
  // 2j in the high nibble; a float4 yields two bytes stored as one uint16.
  uint16_t* dst = reinterpret_cast<uint16_t*>(packed) + blk0 * 16;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int b = i * 16 + (t >> 4);
    if (b >= nblk) continue;
    const float sb = s[i];
    float x[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    uint32_t q[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float xn = sb > 0.0f ? x[e] / sb : 0.0f;
      uint32_t c = 0;
#pragma unroll
      for (int k = 0; k < 15; ++k) c += (xn > tab.thr[k]) ? 1u : 0u;
      q[e] = c;
    }
    const uint32_t b0 = (q[0] << 4) | q[1];
    const uint32_t b1 = (q[2] << 4) | q[3];
    dst[i * 256 + t] = (uint16_t)(b0 | (b1 << 8));
  }
}

hipError_t launch_nf4_quantize(const float* W, uint8_t* packed, uint8_t* codes, float* consts,
                               int64_t numel, hipStream_t stream) {
  const int64_t nb = numel / 64;
  const int64_t ng = (nb + 255) / 256;
  TraceScope ts(KID_QUANTIZE, stream);
  hipLaunchKernelGGL(k_nf4_quantize, dim3((unsigned)ng), dim3(256), 0, stream, W, packed, codes,
                     consts, nb, nf4_table());
  return hipGetLastError();
}

}  // namespace qlora
