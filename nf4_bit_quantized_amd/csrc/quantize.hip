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
// The base weight may also arrive as bf16 or fp16 (the pages quantize an FP16
// model offline): each value is widened exactly to fp32 on load, after which
// the steps are the same, so the result equals quantizing the widened weight.
//
// One workgroup = one second-level group = 256 blocks = 16384 weights.
// 256 threads; thread t loads float4 number i*256 + t (i = 0..15) of the
// group (four 16-bit values, 8 bytes, for a 16-bit weight), so each load
// instruction is a fully coalesced 4 KiB (2 KiB) row; a float4
// belongs to block i*16 + t/16, shared by 16 consecutive lanes, whose absmax
// is reduced with four xor-shuffles inside those 16 lanes.  All sixteen loads
// are issued first; float4 i is quantized and stored as soon as it arrives,
// so the arithmetic of early rows overlaps the loads of later ones.
//
// The index of x = fl32(w / s) is found without the division: a bucket of
// the estimate w * rcp(s) names the one threshold that can matter, and that
// comparison is made exactly in double precision (QuantLut in common.hpp).
// Weights whose block scale is below 2^-64 or above 2^64 are first scaled by
// 2^64 or 2^-64 (exact for every value that can reach a threshold), so the
// reciprocal stays a normal float.  Results are bit-exact: the scale codes use
// IEEE division for s / c_g and rint.  No floating-point contraction.
#pragma clang fp contract(off)

#include <type_traits>

#include "common.hpp"
#include "trace.hpp"

namespace qlora {

// Max over the 16 lanes of a DPP row, left in every lane: swap neighbours,
// swap pairs, mirror the half-rows, mirror the row.
__device__ __forceinline__ float row_max16(float m) {
  auto dpp = [](float v, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), decltype(ctrl)::value,
                                                              0xF, 0xF, false));
  };
  m = fmaxf(m, dpp(m, std::integral_constant<int, 0xB1>{}));   // quad_perm [1,0,3,2]
  m = fmaxf(m, dpp(m, std::integral_constant<int, 0x4E>{}));   // quad_perm [2,3,0,1]
  m = fmaxf(m, dpp(m, std::integral_constant<int, 0x141>{}));  // row_half_mirror
  m = fmaxf(m, dpp(m, std::integral_constant<int, 0x140>{}));  // row_mirror
  return m;
}

// BS: weights per absmax block (64, 128 or 256).  The group's 256 blocks are
// taken in BS/64 passes of 16384 weights each; in a pass, float4 i*256 + t
// belongs to block i*(4096/BS) + t/(BS/4), shared by BS/4 consecutive lanes
// (16, 32 or 64), whose absmax is a DPP row maximum plus one or two xor
// shuffles across rows.
template <int WF, int BS>
__global__ __launch_bounds__(256) void k_nf4_quantize(const void* __restrict__ W,
                                                      uint8_t* __restrict__ packed,
                                                      uint8_t* __restrict__ codes,
                                                      float* __restrict__ consts, int64_t nb,
                                                      QuantLut lut, int dq) {
  static_assert(BS == 64 || BS == 128 || BS == 256, "block size");
  constexpr int NPASS = BS / 64;
  constexpr int LPB = BS / 4;  // lanes per block
  constexpr int kLutWords = (2 * kLutSide + 4) / 4;
  static_assert(kLutWords <= 512, "two words per thread");
  __shared__ uint32_t sh_lut[512];
  __shared__ double sh_mid[16];
  __shared__ float sh_scale[256];
  __shared__ float sh_wmax[4];
  __shared__ __attribute__((aligned(16))) uint16_t sh_packed[NPASS * 16 * 256];  // the group's packed bytes

  const int t = threadIdx.x;
  const int64_t g = blockIdx.x;
  const int64_t blk0 = g * 256;
  const int nblk = (int)((nb - blk0) < 256 ? (nb - blk0) : 256);
  typedef float f4_t __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

  // decision tables: read before the weights, written to LDS after them
  const uint32_t* lw = reinterpret_cast<const uint32_t*>(lut.kidx);
  const uint32_t lut_a = lw[t];
  const uint32_t lut_b = lw[t + 256 < kLutWords ? t + 256 : kLutWords - 1];
  const double mid = lut.mid[t & 15];

  // the group's weights through a buffer resource sized to its blocks, so the
  // float4s of a ragged last group past the end read as zero
  constexpr int EB = WF == kWeightF32 ? 4 : 2;  // bytes per weight
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(W)) + blk0 * BS * EB, (short)0, nblk * BS * EB, 0x00020000);
  float tmax = 0.0f;
#pragma unroll 1
  for (int pass = 0; pass < NPASS; ++pass) {
    f4_t v[16];
    const int f0 = pass * 4096;  // the pass's first float4 in the group
    if constexpr (WF == kWeightF32) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        v[i] = __builtin_bit_cast(f4_t,
                                  __builtin_amdgcn_raw_buffer_load_b128(rsrc, (f0 + i * 256 + t) * 16, 0, 0));
    } else {
      u32x2_t h[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) h[i] = __builtin_amdgcn_raw_buffer_load_b64(rsrc, (f0 + i * 256 + t) * 8, 0, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t u[4] = {h[i].x & 0xFFFFu, h[i].x >> 16, h[i].y & 0xFFFFu, h[i].y >> 16};
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          f[e] = WF == kWeightBf16 ? __builtin_bit_cast(float, u[e] << 16)
                                   : (float)__builtin_bit_cast(_Float16, (uint16_t)u[e]);
        v[i] = f4_t{f[0], f[1], f[2], f[3]};
      }
    }
    if (pass == 0) {
      sh_lut[t] = lut_a;
      sh_lut[t + 256] = lut_b;
      sh_mid[t & 15] = mid;   // 16 threads write each entry, all the same value
      lds_barrier();
    }
    const uint8_t* kidx = reinterpret_cast<const uint8_t*>(sh_lut);

    // per float4: block absmax (4 values per lane, then the block's lanes),
    // indices, two packed bytes as one uint16 (element 2j in the high nibble),
    // staged in LDS and written out below as 16-byte stores
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int b = pass * (4096 / LPB) + i * (256 / LPB) + t / LPB;
      float m = fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w)));
      m = row_max16(m);
      if (LPB >= 32) m = fmaxf(m, __shfl_xor(m, 16));
      if (LPB >= 64) m = fmaxf(m, __shfl_xor(m, 32));
      tmax = fmaxf(tmax, m);
      if ((t % LPB) == 0) sh_scale[b] = m;

      const float pre = m < 0x1p-64f ? 0x1p64f : (m > 0x1p64f ? 0x1p-64f : 1.0f);
      const float rs = m > 0.0f ? __builtin_amdgcn_rcpf(m * pre) : 0.0f;
      const double sd = (double)m;
      const float x[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
      uint32_t q[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ya = (x[e] * pre) * rs;
        const uint32_t bits = __builtin_bit_cast(uint32_t, ya);
        int key = (int)((bits >> 16) & 0x7FFFu) - 0x3C7F;
        key = key < 0 ? 0 : (key > kLutSide - 1 ? kLutSide - 1 : key);
        key += (int)(bits >> 31) * kLutSide;
        const uint32_t k = kidx[key];
        q[e] = k + ((double)x[e] > sd * sh_mid[k] ? 1u : 0u);
      }
      const uint32_t b0 = (q[0] << 4) | q[1];
      const uint32_t b1 = (q[2] << 4) | q[3];
      sh_packed[pass * 4096 + i * 256 + t] = (uint16_t)(b0 | (b1 << 8));
    }
  }

  // group constant c_g = max block scale (all 256 blocks of the group)
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
  if ((t & 63) == 0) sh_wmax[t >> 6] = tmax;
  __syncthreads();
  const float cg = fmaxf(fmaxf(sh_wmax[0], sh_wmax[1]), fmaxf(sh_wmax[2], sh_wmax[3]));

  if (!dq) {  // no second level: the fp32 block scales themselves
    if (t < nblk) consts[blk0 + t] = sh_scale[t];
  } else if (t < nblk) {
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
  if (dq && t == 0) consts[g] = cg;

  // the group's packed bytes (nblk * BS / 2 of them) as 16-byte stores
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(packed + blk0 * (BS / 2));
  const u32x4_t* srcp = reinterpret_cast<const u32x4_t*>(sh_packed);
  for (int c = t; c < nblk * (BS / 32); c += 256) dst[c] = srcp[c];
}

hipError_t launch_nf4_quantize(const void* W, int wformat, uint8_t* packed, uint8_t* codes, float* consts,
                               int64_t numel, int blocksize, int dq, int table, hipStream_t stream) {
  bool ok = false;
  const QuantLut& lut = quant_lut(table, &ok);
  if (!ok) return hipErrorInvalidValue;
  if (wformat != kWeightF32 && wformat != kWeightBf16 && wformat != kWeightF16) return hipErrorInvalidValue;
  if ((blocksize != 64 && blocksize != 128 && blocksize != 256) || numel % blocksize != 0)
    return hipErrorInvalidValue;
  const int64_t nb = numel / blocksize;
  const int64_t ng = (nb + 255) / 256;
  KernelEvents ev(KID_QUANTIZE);
  const dim3 grid((unsigned)ng), block(256);
#define QLORA_QUANT_LAUNCH(WFV, BSV)                                                                            \
  hipExtLaunchKernelGGL((k_nf4_quantize<WFV, BSV>), grid, block, 0, stream, ev.start(), ev.stop(), 0, W, packed, \
                        codes, consts, nb, lut, dq)
#define QLORA_QUANT_BS(WFV)                \
  if (blocksize == 64) QLORA_QUANT_LAUNCH(WFV, 64);   \
  else if (blocksize == 128) QLORA_QUANT_LAUNCH(WFV, 128); \
  else QLORA_QUANT_LAUNCH(WFV, 256)
  if (wformat == kWeightF32) {
    QLORA_QUANT_BS(kWeightF32);
  } else if (wformat == kWeightBf16) {
    QLORA_QUANT_BS(kWeightBf16);
  } else {
    QLORA_QUANT_BS(kWeightF16);
  }
#undef QLORA_QUANT_BS
#undef QLORA_QUANT_LAUNCH
  return hipGetLastError();
}

}  // namespace qlora
