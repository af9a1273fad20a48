// Tiled bf16 MFMA contraction with on-the-fly NF4 restore (gfx950).
//
// C[m][n] = sum_kk Aop[m][kk] * Bop[n][kk], over one or two segments of the
// contraction (the second segment carries the rank-r LoRA term, so it is
// added inside the same fp32 accumulators before the single rounding of the
// output).  Each operand is produced tile by tile into LDS as bf16 with the
// contraction index contiguous ([rows][64], rows padded to 72 elements so
// that 16-byte LDS reads of 32 consecutive rows hit distinct banks).
//
// Restore of the base weight ("QLoRA技术从入门到精通" §3(2): table value times
// the block's stored scale, to a 16-bit float; "【X 长文】..." storage and
// compute paragraph: each block is restored to bf16 just before it enters the
// product and then discarded): the packed nibbles and the 8-bit scale code of
// the 64-weight block are read from memory, the restored scale is
// fl32(code * fl32(c_g / 255)), and each weight becomes bf16(T[q] * s') in LDS.
// It is never written back to memory.  For dX the contraction runs over d_out,
// so each thread restores an 8 x 8 patch (8 rows of W, 8 consecutive k) and
// writes it transposed.
//
// Work split: 256 threads = 4 waves in a WM x WN grid; each wave owns a
// (BM/WM) x (BN/WN) sub-tile made of 32 x 32 MFMA tiles
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation).  Optional split of the
// contraction across grid.z writes fp32 partials that a separate kernel sums
// in a fixed order (deterministic, no atomics).
#include "gemm.hpp"
#include "trace.hpp"

namespace qlora {

namespace {

constexpr int BK = 64;
constexpr int LDS_LD = BK + 8;  // bf16 elements per LDS row

__device__ __forceinline__ uint32_t nibble(uint32_t w, int e) {
  // element e (0..7) of a little-endian word: byte e/2, high nibble first
  return (w >> (8 * (e >> 1) + ((e & 1) ? 0 : 4))) & 0xFu;
}

__device__ __forceinline__ uint4 pack8(const uint16_t* e) {
  uint4 v;
  v.x = (uint32_t)e[0] | ((uint32_t)e[1] << 16);
  v.y = (uint32_t)e[2] | ((uint32_t)e[3] << 16);
  v.z = (uint32_t)e[4] | ((uint32_t)e[5] << 16);
  v.w = (uint32_t)e[6] | ((uint32_t)e[7] << 16);
  return v;
}

__device__ __forceinline__ void unpack8(uint4 v, uint16_t* e) {
  e[0] = (uint16_t)(v.x & 0xFFFF); e[1] = (uint16_t)(v.x >> 16);
  e[2] = (uint16_t)(v.y & 0xFFFF); e[3] = (uint16_t)(v.y >> 16);
  e[4] = (uint16_t)(v.z & 0xFFFF); e[5] = (uint16_t)(v.z >> 16);
  e[6] = (uint16_t)(v.w & 0xFFFF); e[7] = (uint16_t)(v.w >> 16);
}

__device__ __forceinline__ int64_t src_kk(const Operand& op, int64_t kk) {
  return op.kk_mod ? kk % op.kk_mod : kk;
}

// Fill S[ROWS][LDS_LD] with Op[row0 + r][kt*64 + c] as bf16 bits.  KIND is
// the operand kind when known at compile time, or -1 to dispatch on op.kind.
template <int ROWS, int KIND>
__device__ __forceinline__ void load_tile(const Operand& op, int64_t row0, int64_t kt,
                                          uint16_t* __restrict__ S, const float* __restrict__ lut) {
  const int tid = threadIdx.x;
  const int64_t k0 = kt * BK;
  switch (KIND >= 0 ? KIND : op.kind) {
    case OP_BF16_K: {
      const uint16_t* p = static_cast<const uint16_t*>(op.p);
      const bool vec = op.kk_mod == 0 && (op.ld & 7) == 0 && (reinterpret_cast<uintptr_t>(p) & 15) == 0;
      for (int c = tid; c < ROWS * 8; c += 256) {
        const int r = c >> 3, kc = (c & 7) * 8;
        const int64_t row = row0 + r, kk = k0 + kc;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < op.rows) {
          if (vec && kk + 8 <= op.kdim) {
            v = *reinterpret_cast<const uint4*>(p + row * op.ld + kk);
          } else {
            uint16_t e[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
              e[i] = (kk + i < op.kdim) ? p[row * op.ld + src_kk(op, kk + i)] : (uint16_t)0;
            v = pack8(e);
          }
        }
        *reinterpret_cast<uint4*>(S + r * LDS_LD + kc) = v;
      }
      break;
    }
    case OP_BF16_T: {
      const uint16_t* p = static_cast<const uint16_t*>(op.p);
      const bool vec = (op.ld & 7) == 0 && (reinterpret_cast<uintptr_t>(p) & 15) == 0;
      for (int c = tid; c < ROWS; c += 256) {
        const int rb = c >> 3, cb = c & 7;
        const int64_t r8 = row0 + rb * 8, kk8 = k0 + cb * 8;
        uint16_t e[8][8];  // e[i][j] = Op[r8 + j][kk8 + i]
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int64_t kk = kk8 + i;
          uint4 v = make_uint4(0, 0, 0, 0);
          if (kk < op.kdim && r8 < op.rows) {
            const uint16_t* src = p + src_kk(op, kk) * op.ld + r8;
            if (vec && r8 + 8 <= op.rows) {
              v = *reinterpret_cast<const uint4*>(src);
            } else {
              uint16_t t8[8];
#pragma unroll
              for (int j = 0; j < 8; ++j) t8[j] = (r8 + j < op.rows) ? src[j] : (uint16_t)0;
              v = pack8(t8);
            }
          }
          unpack8(v, e[i]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          uint16_t o[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) o[i] = e[i][j];
          *reinterpret_cast<uint4*>(S + (rb * 8 + j) * LDS_LD + cb * 8) = pack8(o);
        }
      }
      break;
    }
    case OP_NF4_K: {
      const uint8_t* pk = static_cast<const uint8_t*>(op.p);
      const int64_t K = op.ld, kb_row = K / 64;
      for (int c = tid; c < ROWS * 2; c += 256) {
        const int r = c >> 1, h = c & 1;
        const int64_t n = row0 + r, k = k0 + h * 32;
        uint32_t out[16];
        if (n < op.rows && k < op.kdim) {
          const uint4 pv = *reinterpret_cast<const uint4*>(pk + n * (K / 2) + k / 2);
          const int64_t blk = n * kb_row + kt;
          const float sc = restored_scale(op.codes[blk], op.consts[blk >> 8]);
          const uint32_t wv[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
          for (int b = 0; b < 16; ++b) {
            const uint32_t byte = (wv[b >> 2] >> (8 * (b & 3))) & 0xFFu;
            out[b] = pack_bf16x2(lut[byte >> 4] * sc, lut[byte & 15u] * sc);
          }
        } else {
#pragma unroll
          for (int b = 0; b < 16; ++b) out[b] = 0;
        }
        uint4* dst = reinterpret_cast<uint4*>(S + r * LDS_LD + h * 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = make_uint4(out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]);
      }
      break;
    }
    case OP_NF4_T: {
      const uint8_t* pk = static_cast<const uint8_t*>(op.p);
      const int64_t K = op.ld, kb_row = K / 64;
      for (int c = tid; c < ROWS; c += 256) {
        const int rb = c >> 3, cb = c & 7;
        const int64_t k8 = row0 + rb * 8;  // output rows are k (d_in)
        const int64_t n8 = k0 + cb * 8;    // contraction runs over n (d_out)
        float vals[8][8];                  // vals[i][e] = W_hat[n8 + i][k8 + e]
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int64_t n = n8 + i;
          if (n < op.kdim && k8 < op.rows) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(pk + n * (K / 2) + k8 / 2);
            const int64_t blk = n * kb_row + k8 / 64;
            const float sc = restored_scale(op.codes[blk], op.consts[blk >> 8]);
#pragma unroll
            for (int e = 0; e < 8; ++e) vals[i][e] = lut[nibble(w, e)] * sc;
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) vals[i][e] = 0.0f;
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint4 o = make_uint4(pack_bf16x2(vals[0][j], vals[1][j]), pack_bf16x2(vals[2][j], vals[3][j]),
                                     pack_bf16x2(vals[4][j], vals[5][j]), pack_bf16x2(vals[6][j], vals[7][j]));
          *reinterpret_cast<uint4*>(S + (rb * 8 + j) * LDS_LD + cb * 8) = o;
        }
      }
      break;
    }
    default: {
      for (int c = tid; c < ROWS * 8; c += 256)
        *reinterpret_cast<uint4*>(S + (c >> 3) * LDS_LD + (c & 7) * 8) = make_uint4(0, 0, 0, 0);
      break;
    }
  }
}

template <int BM, int BN, int WM, int WN, int KA, int KB>
__device__ __forceinline__ void gemm_body(const GemmParams& P, const Nf4Table& tab) {
  static_assert(WM * WN == 4, "4 waves");
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
  static_assert(TM >= 1 && TN >= 1, "wave tile at least 32 x 32");

  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDS_LD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDS_LD];
  __shared__ float lut[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int z = blockIdx.z;

  if (tid < 16) lut[tid] = tab.level[tid];

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int64_t nt0 = P.seg[0].ktiles;
  const int64_t total = nt0 + (P.nseg > 1 ? P.seg[1].ktiles : 0);
  const int64_t t_begin = (int64_t)z * P.tiles_per_split;
  const int64_t t_end = t_begin + P.tiles_per_split < total ? t_begin + P.tiles_per_split : total;

  for (int64_t t = t_begin; t < t_end; ++t) {
    __syncthreads();
    if (t < nt0) {
      load_tile<BM, KA>(P.seg[0].a, m0, t, As, lut);
      load_tile<BN, KB>(P.seg[0].b, n0, t, Bs, lut);
    } else {
      load_tile<BM, -1>(P.seg[1].a, m0, t - nt0, As, lut);
      load_tile<BN, -1>(P.seg[1].b, n0, t - nt0, Bs, lut);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t a[TM], b[TN];
      const int kofs = ks * 16 + (lane >> 5) * 8;
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(As + ((wm * TM + i) * 32 + (lane & 31)) * LDS_LD + kofs);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(Bs + ((wn * TN + j) * 32 + (lane & 31)) * LDS_LD + kofs);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }

  // epilogue: lane holds column (lane & 31) and rows 8*(v/4) + 4*(lane/32) + v%4
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t col = n0 + (wn * TN + j) * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + (wm * TM + i) * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < P.M && col < P.N) {
          if (P.out_kind == OUT_BF16)
            static_cast<uint16_t*>(P.out)[row * P.ldo + col] = f32_to_bf16_bits(acc[i][j][v]);
          else
            static_cast<float*>(P.out)[(int64_t)z * P.split_stride + row * P.ldo + col] = acc[i][j][v];
        }
      }
    }
  }
}

// Adapter products and anything else: operand kinds read at run time.
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256) void k_lowrank_gemm(GemmParams P, Nf4Table tab) {
  gemm_body<BM, BN, WM, WN, -1, -1>(P, tab);
}

}  // namespace

// Tile shapes: 0 = 128x128 (2x2 waves), 1 = 32x128 (1x4), 2 = 128x32 (4x1), 3 = 64x64 (2x2).
int gemm_tile_config(int64_t M, int64_t N) {
  if (M <= 32) return 1;
  if (N <= 32) return 2;
  if (M <= 64 || N <= 64) return 3;
  return 0;
}

void gemm_tile_shape(int cfg, int* bm, int* bn) {
  static const int S[4][2] = {{128, 128}, {32, 128}, {128, 32}, {64, 64}};
  *bm = S[cfg][0];
  *bn = S[cfg][1];
}

hipError_t launch_gemm(const GemmParams& p, hipStream_t stream, int kernel_id) {
  const int cfg = gemm_tile_config(p.M, p.N);
  int bm, bn;
  gemm_tile_shape(cfg, &bm, &bn);
  const dim3 grid((unsigned)((p.N + bn - 1) / bn), (unsigned)((p.M + bm - 1) / bm), (unsigned)p.nsplit);
  const Nf4Table& tab = nf4_table();
  TraceScope ts(kernel_id, stream);
  switch (cfg) {
    case 0: hipLaunchKernelGGL((k_lowrank_gemm<128, 128, 2, 2>), grid, dim3(256), 0, stream, p, tab); break;
    case 1: hipLaunchKernelGGL((k_lowrank_gemm<32, 128, 1, 4>), grid, dim3(256), 0, stream, p, tab); break;
    case 2: hipLaunchKernelGGL((k_lowrank_gemm<128, 32, 4, 1>), grid, dim3(256), 0, stream, p, tab); break;
    default: hipLaunchKernelGGL((k_lowrank_gemm<64, 64, 2, 2>), grid, dim3(256), 0, stream, p, tab); break;
  }
  return hipGetLastError();
}

}  // namespace qlora
