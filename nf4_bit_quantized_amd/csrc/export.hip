// Export of the restored weight, and of the weight with the adapter merged in.
//
// "QLoRA技术从入门到精通" §3(2): the 4-bit weight is restored to a 16-bit float
// (table value times the block's restored scale).  "LoRA 与 QLoRA：把大模型微调
// 拆成可负担的工程" §3: after training the update can be merged into the
// weight, W + (alpha / r) B A.  "【X 长文】LoRA 与 QLoRA：用一块 GPU 微调大模型",
// QLoRA section: with a 4-bit base the trained A and B cannot be added to the
// 4-bit weight; they are merged into the restored 16-bit weight.
//
//   dequantize:  W_out = W_hat = bf16_rne(fl32(T[q] * s'))       (bit-exact)
//   merge:       W_out = bf16_rne( fl32( W_hat + fl32(s * (B A)) ) ),  s = fl32(alpha / r)
//
// Dequantize: a flat pass, four 16-weight pairs of packed words per thread
// (a pair shares one block and its table), all loads issued before any
// restore, 32-byte stores.
//
// Merge: a workgroup owns a 128-column block of W for a run of 64-row tiles
// (three workgroups per CU fill the GPU once), 256 threads; the block's slice
// of A is staged in LDS once, and the next tile's packed words, codes,
// constants and B rows are loaded while the current tile is formed.  A
// tile's rank-r term runs on v_mfma_f32_16x16x32_bf16.  Wave w
// takes rows 16w .. 16w+15.  Operand A is rows of B ([N][r]; lane l: row
// l % 16, j = 8(l/16) ..); operand B is the tile's columns of A ([r][K]),
// copied to LDS once and read with ds_read_b64_tr_b16 (within a 16-lane
// group, source lane s points at row kb + s/4, columns c0 + 4(s%4); lane i
// receives rows kb .. kb+3 of column c0 + i).  r is padded to a multiple of 32
// with zeros.  s times the fp32 result is written to an LDS tile.
//
// Then every thread restores two pairs of packed words of the tile (8
// weights each, the restore of the fused products; the two words of a pair
// share a block and its table), adds the LDS term when merging, rounds once
// to bf16 and writes 32 bytes; a row's 8 pairs are 8 consecutive threads, so
// loads and stores are coalesced.  The A tile is sized to the rank (dynamic
// LDS), so short ranks leave room for more workgroups per CU.
#include "common.hpp"
#include "restore.hpp"
#include "trace.hpp"

namespace qlora {

namespace {

constexpr int TR = 64, TC = 128;  // tile rows (weight rows) and columns
constexpr int LDA = TC + 16;      // bf16 row of the A tile in LDS
constexpr int LDD = TC + 4;       // fp32 row of the rank-r term in LDS
constexpr int MAX_R = 128;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) uint16_t lds_u16_t;

struct ExportParams {
  const uint8_t* packed;
  const uint8_t* codes;
  const float* consts;
  int64_t N, K;
  const uint16_t* A;  // [r][K] bf16 (merge only)
  const uint16_t* B;  // [N][r] bf16 (merge only)
  int r;
  float s;
  uint16_t* W;        // [N][K] bf16 out
  Nf4Table tab;
  int bshift;         // log2(weights per absmax block / 64)
  int dq;             // 1: codes + group constants; 0: consts holds the fp32 block scales
};

// One 64-row tile's data for the merge: the thread's two pairs of packed
// words with their codes and constants, and the wave's B fragments (its 16
// rows, 32 ranks per fragment).
struct MergeTile {
  uint2 w[2];
  uint32_t code[2];
  float cg[2];
  u16x8_t b[MAX_R / 32];
};

__global__ __launch_bounds__(256) void k_merge(ExportParams P, int tpw) {
  // dynamic LDS: D [TR][LDD] fp32, then the A tile [rpad][LDA] bf16
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  float* D = dyn;
  uint16_t* At = reinterpret_cast<uint16_t*>(dyn + TR * LDD);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, g = lane >> 4;
  const int64_t k0 = (int64_t)blockIdx.x * TC;
  const int64_t ntile = P.N / TR;
  const int64_t t0 = (int64_t)blockIdx.y * tpw;
  const int64_t t1 = t0 + tpw < ntile ? t0 + tpw : ntile;
  const int rpad = (P.r + 31) & ~31;

  // tile t's loads (pairs past K read the row's first pair and are not stored)
  auto load = [&](MergeTile& R, int64_t t) {
    const int64_t i0 = t * TR;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int d = tid + 256 * q;
      const int64_t n = i0 + (d >> 3), kc = k0 + 16 * (d & 7);
      const int64_t e0 = n * P.K + (kc < P.K ? kc : 0);
      R.w[q] = *reinterpret_cast<const uint2*>(P.packed + e0 / 2);
      const int64_t blk = (e0 / 64) >> P.bshift;
      R.code[q] = P.dq ? P.codes[blk] : 0u;
      R.cg[q] = P.consts[P.dq ? blk >> 8 : blk];
    }
    const int64_t brow = i0 + 16 * wave + i16;
#pragma unroll
    for (int jb = 0; jb < MAX_R / 32; ++jb) {
      const int js = 32 * jb;
      if (js >= rpad) break;
      if ((P.r & 7) == 0) {
        const int j0 = js + 8 * g;
        R.b[jb] = j0 < P.r ? *reinterpret_cast<const u16x8_t*>(P.B + brow * P.r + j0) : u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int jj = js + 8 * g + q;
          R.b[jb][q] = jj < P.r ? P.B[brow * P.r + jj] : (uint16_t)0;
        }
      }
    }
  };

  MergeTile cur, nxt;
  load(cur, t0);
  // A[j][k0 .. k0+127], zero for j >= r or columns past K: staged once for every tile
  for (int c = tid; c < rpad * (TC / 8); c += 256) {
    const int j = c / (TC / 8), cc = (c % (TC / 8)) * 8;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (j < P.r && k0 + cc < P.K) v = *reinterpret_cast<const u32x4_t*>(P.A + (int64_t)j * P.K + k0 + cc);
    *reinterpret_cast<u32x4_t*>(At + j * LDA + cc) = v;
  }
  __syncthreads();
  const lds_u16_t* at = (const lds_u16_t*)At;
  for (int64_t t = t0; t < t1; ++t) {
    if (t + 1 < t1) load(nxt, t + 1);  // the next tile's data arrives while this one is formed
    f32x4_t acc[TC / 16];
#pragma unroll
    for (int ct = 0; ct < TC / 16; ++ct) acc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jb = 0; jb < MAX_R / 32; ++jb) {
      const int js = 32 * jb;
      if (js >= rpad) break;
      const int row = js + 8 * g + (i16 >> 2);
#pragma unroll
      for (int ct = 0; ct < TC / 16; ++ct) {
        const int col = 16 * ct + 4 * (i16 & 3);
        const u16x4_t lo = __builtin_bit_cast(
            u16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(at + row * LDA + col)));
        const u16x4_t hi = __builtin_bit_cast(
            u16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(at + (row + 4) * LDA + col)));
        const u16x8_t b = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, cur.b[jb]),
                                                          __builtin_bit_cast(bf16x8_t, b), acc[ct], 0, 0, 0);
      }
    }
    // C layout: lane l, value v holds row 4(l/16) + v, column l % 16 of the tile
#pragma unroll
    for (int ct = 0; ct < TC / 16; ++ct)
#pragma unroll
      for (int v = 0; v < 4; ++v) D[(16 * wave + 4 * g + v) * LDD + 16 * ct + i16] = P.s * acc[ct][v];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int d = tid + 256 * q;
      const int row = d >> 3, cp = (d & 7) * 2;  // words cp, cp + 1 of the row (one block)
      const int64_t n = t * TR + row, kc = k0 + 8 * cp;
      if (kc >= P.K) continue;
      const int64_t e0 = n * P.K + kc;  // element index of the pair's first weight
      const RestoreTab tb = make_tab(P.tab, P.dq ? restored_scale(cur.code[q], cur.cg[q]) : cur.cg[q]);
      uint32_t o[8];
      restore8(cur.w[q].x, tb, o);
      restore8(cur.w[q].y, tb, o + 4);
      const float* dr = D + row * LDD + 8 * cp;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        o[e] = pack_bf16x2(bf16_bits_to_f32(o[e] & 0xFFFFu) + dr[2 * e], bf16_bits_to_f32(o[e] >> 16) + dr[2 * e + 1]);
      uint4* dst = reinterpret_cast<uint4*>(P.W + e0);
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
    __syncthreads();  // D is read before the next tile writes it
    cur = nxt;
  }
}

// Dequantize only: pairs p = 16-weight runs in element order (packed bytes
// 8p .. 8p+7, block 16p / blocksize).
constexpr int DQ_PER = 4;
__global__ __launch_bounds__(256) void k_dequant(ExportParams P) {
  const int64_t npairs = P.N * P.K / 16;
  const int64_t p0 = ((int64_t)blockIdx.x * 256 * DQ_PER) + threadIdx.x;
  uint2 w[DQ_PER];
  uint32_t code[DQ_PER];
  float cg[DQ_PER];
#pragma unroll
  for (int q = 0; q < DQ_PER; ++q) {
    const int64_t p = p0 + 256 * q;
    const int64_t pc = p < npairs ? p : npairs - 1;
    w[q] = *reinterpret_cast<const uint2*>(P.packed + 8 * pc);
    const int64_t blk = pc >> (2 + P.bshift);
    code[q] = P.dq ? P.codes[blk] : 0u;
    cg[q] = P.consts[P.dq ? blk >> 8 : blk];
  }
#pragma unroll
  for (int q = 0; q < DQ_PER; ++q) {
    const int64_t p = p0 + 256 * q;
    if (p >= npairs) break;
    const RestoreTab t = make_tab(P.tab, P.dq ? restored_scale(code[q], cg[q]) : cg[q]);
    uint32_t o[8];
    restore8(w[q].x, t, o);
    restore8(w[q].y, t, o + 4);
    uint4* dst = reinterpret_cast<uint4*>(P.W + 16 * p);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

}  // namespace

hipError_t launch_export(const uint8_t* packed, const uint8_t* codes, const float* consts, int64_t N, int64_t K,
                         int r, float s, const uint16_t* A, const uint16_t* B, uint16_t* W, int table,
                         int bshift, int dq, hipStream_t stream) {
  if (N % TR != 0 || K % 64 != 0 || r < 0 || r > MAX_R || bshift < 0 || bshift > 2) return hipErrorInvalidValue;
  ExportParams P;
  P.packed = packed; P.codes = codes; P.consts = consts;
  P.N = N; P.K = K;
  P.A = A; P.B = B; P.r = r; P.s = s;
  P.W = W;
  P.tab = level_table(table);
  P.bshift = bshift;
  P.dq = dq;
  KernelEvents ev(KID_EXPORT);
  if (r > 0) {
    // runs of row tiles per workgroup: three workgroups per CU fill the 256 CUs once
    const int64_t ntile = N / TR, ncol = (K + TC - 1) / TC;
    int64_t groups = 768 / ncol;
    groups = groups < 1 ? 1 : (groups > ntile ? ntile : groups);
    const int tpw = (int)((ntile + groups - 1) / groups);
    const dim3 mgrid((unsigned)ncol, (unsigned)((ntile + tpw - 1) / tpw));
    const size_t lds = (size_t)TR * LDD * 4 + (size_t)((r + 31) & ~31) * LDA * 2;
    hipExtLaunchKernelGGL(k_merge, mgrid, dim3(256), (uint32_t)lds, stream, ev.start(), ev.stop(), 0, P, tpw);
  } else {
    const int64_t npairs = N * K / 16;
    const unsigned g = (unsigned)((npairs + 256 * DQ_PER - 1) / (256 * DQ_PER));
    hipExtLaunchKernelGGL(k_dequant, dim3(g), dim3(256), 0, stream, ev.start(), ev.stop(), 0, P);
  }
  return hipGetLastError();
}

}  // namespace qlora
