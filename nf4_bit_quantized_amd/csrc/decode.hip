// Forward for few tokens (T <= 16): stream the packed weight once.
//
// With at most 16 tokens the product X W_hat^T is bound by reading the packed
// nibbles and scale codes from HBM ("QLoRA技术从入门到精通" §3(2): the 4-bit
// weight is restored block by block at compute time and discarded).
//
// Workgroup: 4 waves, 64 weight rows, one slice of the contraction, walked in
// stages of 8 blocks (512 weights per row).  A stage is loaded with long runs
// per row -- each load instruction covers 4 rows x 256 bytes of packed data,
// one token row of X (1 KB) or the 8 scale codes of 16 rows -- into registers
// two or three stages ahead of use (fewer tokens, fewer X registers, deeper),
// written to one of two LDS buffers one stage ahead,
// and multiplied from LDS.  (Spreading each load instruction over 32 rows of
// 32 bytes, the MFMA operand layout, reads HBM at about half the rate.)
//
// Restore: a packed byte holding levels (q_hi, q_lo) is looked up in a
// 256-entry LDS table of the pairs bf16(T[q_hi]), bf16(T[q_lo]) in element
// order.  The block scale is applied to the MFMA result instead: the four
// v_mfma_f32_32x32x16_bf16 of one block of 32 rows cover exactly that block's
// 64 weights of each row, so their sum is multiplied by the row's restored
// scale s' = fl32(code) * fl32(c_g / 255) and added to an fp32 accumulator.
// (This differs from rounding T[q] * s' to bf16 by at most one bf16 rounding
// of each weight.)  fl32(c_g / 255) is computed once per row and group, into
// an LDS table, before the stages start.  MFMA operands: X is the 32 x 16 A
// operand (token rows >= T read a zero row), the restored weight the 16 x 32
// B operand; in MFMA j of a block, lane group g supplies weights 32g+8j..+8.
// Wave w multiplies blocks 2w and 2w+1 of every stage for all 64 rows.
//
// Rank-r term: the workgroups of the first contraction slice add
// s (X A^T) B^T through the same MFMA, over the 2r hi/lo columns of s U
// (zero-padded to a multiple of 64), as the dense kernels do.
//
// The four waves' sums are added in LDS in a fixed order.  One slice: bf16 Y
// is written directly; several slices: fp32 partials, summed in slice order by
// k_decode_reduce.
#include "common.hpp"
#include "trace.hpp"

namespace qlora {

namespace {

constexpr int ROWS = 64;        // weight rows per workgroup (two 32-row MFMA tiles)
constexpr int WAVES = 4;
constexpr int SB = 8;           // blocks per stage
constexpr int MAXG = 5;         // groups of 256 blocks a row can touch inside one slice
constexpr int WLD = SB * 32 + 16;       // LDS row of packed bytes (256 + 16 pad)
constexpr int XLD = SB * 64 * 2 + 16;   // LDS row of X bytes (1024 + 16 pad)
constexpr int XROWS = 17;               // 16 token rows + one zero row

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

struct DecodeParams {
  const uint8_t* packed;
  const uint8_t* codes;
  const float* consts;
  const uint16_t* X;
  int64_t T, N, K;
  const uint16_t* Us;  // hi/lo pair of s*U, [T][ldh], zero past 2r (unused when r == 0)
  int64_t ldh;
  const uint16_t* B;   // [N][r]
  int r;
  int nsplit;
  int64_t per;         // blocks per contraction slice (a multiple of SB)
  uint16_t* Y;         // [T][N] (one slice)
  float* part;         // [nsplit][T][N] (several slices)
  float level[16];
};

// One stage's loads for one wave: packed bytes of 16 rows (4 per load), XR
// token rows of X (rows >= T read as zero), the stage's scale codes of 16 rows.
template <int XR>
struct StageRegs {
  u32x4_t w[4];
  u32x4_t x[XR];
  u32x2_t code;
};

struct Cursor {
  __amdgpu_buffer_rsrc_t rw, rx, rc;
  uint32_t woff;       // this lane's packed-byte offset for stage 0, load 0
  uint32_t wrow_step;  // bytes between the loads' row groups (4 rows)
  uint32_t xoff;       // this lane's X byte offset for stage 0, token row = wave
  uint32_t xrow_step;  // bytes between the token rows a wave loads (4 rows apart)
  uint32_t coff;       // this lane's code offset for stage 0
};

struct Smem {
  uint8_t w[2][ROWS * WLD];       // packed bytes, [row][256 B]
  uint8_t x[2][XROWS * XLD];      // X, [token][1 KB]; row 16 stays zero
  uint8_t code[2][ROWS * SB];     // scale codes, [row][block]
  float ratio[ROWS][MAXG];        // fl32(c_g / 255) of the row's groups in this slice
  uint32_t lut[256];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int64_t bytes) {
  const int32_t n = bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0 : (int32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}

// CODES4: the rows' code runs start on 4-byte boundaries (K % 256 == 0), so a
// stage's 8 codes of a row are one 8-byte load; otherwise eight byte loads.
template <bool CODES4, int XR>
__device__ __forceinline__ void load_stage(StageRegs<XR>& R, const Cursor& c, uint32_t blk0) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    R.w[i] = __builtin_amdgcn_raw_buffer_load_b128(c.rw, c.woff + i * c.wrow_step, blk0 * 32u, 0);
#pragma unroll
  for (int i = 0; i < XR; ++i)
    R.x[i] = __builtin_amdgcn_raw_buffer_load_b128(c.rx, c.xoff + i * c.xrow_step, blk0 * 128u, 0);
  if (CODES4) {
    R.code = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(c.rc, c.coff, blk0, 0));
  } else {
    uint32_t b[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) b[q] = __builtin_amdgcn_raw_buffer_load_b8(c.rc, c.coff + q, blk0, 0);
    R.code = u32x2_t{b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24), b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24)};
  }
}

// Registers -> LDS buffer: this wave's 16 rows of packed bytes, its XR token
// rows of X (wave, wave + 4, ...) and the codes of its 16 rows.
template <int XR>
__device__ __forceinline__ void store_stage(const StageRegs<XR>& R, Smem& sm, int buf, int wave, int lane) {
  // load i holds rows wave*16 + 4i + lane/16, bytes (lane%16)*16
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wave * 16 + 4 * i + (lane >> 4);
    *reinterpret_cast<u32x4_t*>(&sm.w[buf][row * WLD + (lane & 15) * 16]) = R.w[i];
  }
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const int t = wave + 4 * i;
    *reinterpret_cast<u32x4_t*>(&sm.x[buf][t * XLD + lane * 16]) = R.x[i];
  }
  if (lane < 16) *reinterpret_cast<u32x2_t*>(&sm.code[buf][(wave * 16 + lane) * SB]) = R.code;
}

__device__ __forceinline__ bf16x8_t lookup8(uint32_t d, const uint32_t* __restrict__ lut) {
  u32x4_t o;
  o.x = lut[d & 0xFFu];
  o.y = lut[(d >> 8) & 0xFFu];
  o.z = lut[(d >> 16) & 0xFFu];
  o.w = lut[d >> 24];
  return __builtin_bit_cast(bf16x8_t, o);
}

// XR: token rows of X each wave stages (X holds up to 4 * XR tokens);
// DEPTH: stages loaded ahead of use (register sets: DEPTH + 1).
template <bool CODES4, int XR, int DEPTH>
__global__ __launch_bounds__(256) void k_decode(DecodeParams P) {
  __shared__ __attribute__((aligned(16))) Smem sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 31, g = lane >> 5;
  const int64_t n0 = (int64_t)blockIdx.x * ROWS;
  const int z = blockIdx.y;
  const int64_t nbk = P.K / 64;
  const int64_t kb = (int64_t)z * P.per;
  const int64_t ke = kb + P.per < nbk ? kb + P.per : nbk;
  const int nst = kb < ke ? (int)((ke - kb + SB - 1) / SB) : 0;

  // byte table, zero X rows, per-row ratios c_g / 255 of the groups this slice touches
  sm.lut[tid] = pack_bf16x2(P.level[tid >> 4], P.level[tid & 15]);
  for (int i = tid; i < XLD / 4; i += 256) {
    reinterpret_cast<uint32_t*>(&sm.x[0][16 * XLD])[i] = 0u;
    reinterpret_cast<uint32_t*>(&sm.x[1][16 * XLD])[i] = 0u;
  }
  const int64_t ngroups = (P.N * nbk + 255) / 256;
  for (int i = tid; i < ROWS * MAXG; i += 256) {
    const int row = i / MAXG, k = i % MAXG;
    const int64_t gi = (((n0 + row) * nbk + kb) >> 8) + k;
    sm.ratio[row][k] = gi < ngroups ? P.consts[gi] / 255.0f : 0.0f;
  }

  Cursor c;
  c.rw = rsrc(P.packed, P.N * P.K / 2);
  c.rx = rsrc(P.X, P.T * P.K * 2);
  c.rc = rsrc(P.codes, P.N * nbk);
  c.woff = (uint32_t)((n0 + wave * 16 + (lane >> 4)) * (P.K / 2) + (lane & 15) * 16);
  c.wrow_step = (uint32_t)(4 * (P.K / 2));
  c.xoff = (uint32_t)((int64_t)wave * P.K * 2 + lane * 16);  // token rows >= T lie past the end: zero
  c.xrow_step = (uint32_t)(4 * P.K * 2);
  c.coff = (uint32_t)((n0 + wave * 16 + (lane & 15)) * nbk);

  float acc[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[i][v] = 0.0f;

  // stage s covers blocks kb + s*SB ...; loads outside [0, nst) repeat an end stage
  auto blk_of = [&](int s) {
    const int j = s < 0 ? 0 : (s < nst ? s : nst - 1);
    return (uint32_t)(kb + (int64_t)SB * j);
  };
  auto compute = [&](int buf, uint32_t blk0) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int b = 2 * wave + bb;                  // block inside the stage
      const uint32_t blk = blk0 + (uint32_t)b;      // block inside the row
      const bool live = blk < (uint32_t)ke;         // blocks past the slice count zero
      const int t = nl < P.T ? nl : 16;  // rows 4*XR .. 15 are never written: T <= 4*XR
      bf16x8_t xf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xf[j] = *reinterpret_cast<const bf16x8_t*>(&sm.x[buf][t * XLD + (64 * b + 32 * g + 8 * j) * 2]);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = 32 * i + nl;
        const u32x4_t wv = *reinterpret_cast<const u32x4_t*>(&sm.w[buf][row * WLD + 32 * b + 16 * g]);
        const uint32_t code = sm.code[buf][row * SB + b];
        const int64_t rb = (n0 + row) * nbk;
        int gk = (int)(((rb + blk) >> 8) - ((rb + kb) >> 8));
        gk = gk < MAXG ? gk : MAXG - 1;
        const float sc = live ? (float)code * sm.ratio[row][gk] : 0.0f;
        f32x16_t cblk = {};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          cblk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf[j], lookup8(wv[j], sm.lut), cblk, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[i][v] = fmaf(sc, cblk[v], acc[i][v]);
      }
    }
  };

  if (nst > 0) {
    // Stage x lives in register set x mod (DEPTH + 1): loaded at step x - DEPTH,
    // written to LDS buffer x & 1 at step x - 1, multiplied at step x.  The
    // first period only loads (its stores and multiplies are skipped by uniform
    // tests), so the sets live in the same registers from the first load on.
    StageRegs<XR> R[DEPTH + 1];
    int s = -(DEPTH + 1);
    for (; s + DEPTH + 1 <= nst; s += DEPTH + 1) {
#pragma unroll
      for (int d = 0; d <= DEPTH; ++d) {
        const int st = s + d;  // stage multiplied in this step
        load_stage<CODES4, XR>(R[(d + DEPTH) % (DEPTH + 1)], c, blk_of(st + DEPTH));
        asm volatile("" ::: "memory");  // keep the loads in stage order (waits count in issue order)
        if (st + 1 >= 0) store_stage(R[(d + 1) % (DEPTH + 1)], sm, (st + 1) & 1, wave, lane);
        if (st >= 0) compute(st & 1, blk_of(st));
        lds_barrier();
      }
    }
    // the last stages: stage s is in LDS, stages s+1 .. s+DEPTH-1 in R[1 ..]
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int st = s + d;
      if (st < nst) {
        if (d + 1 < DEPTH && st + 1 < nst) store_stage(R[d + 1], sm, (st + 1) & 1, wave, lane);
        compute(st & 1, blk_of(st));
      }
      lds_barrier();
    }
  }
  __syncthreads();

  // rank-r term (first slice only): wave i adds it for tile i
  if (P.r > 0 && z == 0 && wave < 2) {
    const int i = wave;
    const int64_t n = n0 + 32 * i + nl;
    const __amdgpu_buffer_rsrc_t ru = rsrc(P.Us, P.T * P.ldh * 2);
    f32x16_t ct = {};
#pragma unroll
    for (int v = 0; v < 8; ++v) ct[v] = acc[i][v];
    for (int64_t kk = 0; kk < P.ldh; kk += 16) {
      const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(ru, (uint32_t)(((int64_t)nl * P.ldh + kk + 8 * g) * 2), 0, 0);
      const uint32_t j0 = (uint32_t)((kk + 8 * g) % P.r);
      u32x4_t b;
      if ((P.r & 7) == 0) {
        b = *reinterpret_cast<const u32x4_t*>(P.B + n * P.r + j0);
      } else {
        uint16_t e[8];
        for (int q = 0; q < 8; ++q) e[q] = P.B[n * P.r + (j0 + q) % (uint32_t)P.r];
        b = u32x4_t{e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16), e[4] | ((uint32_t)e[5] << 16),
                    e[6] | ((uint32_t)e[7] << 16)};
      }
      ct = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                    ct, 0, 0, 0);
    }
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[i][v] = ct[v];
  }

  // add the four waves' sums (in the packed-byte buffers, free by now); lane
  // l, value v of tile i holds token 8(v/4) + 4(l/32) + v%4 of row 32i + l%32
  float* red = reinterpret_cast<float*>(&sm.w[0][0]);  // [wave][tile][v][lane], 16 KB
  static_assert(sizeof(sm.w) >= WAVES * 2 * 8 * 64 * 4, "reduction fits in the packed-byte buffers");
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 8; ++v) red[((wave * 2 + i) * 8 + v) * 64 + lane] = acc[i][v];
  __syncthreads();
  for (int o = tid; o < 16 * ROWS; o += 256) {
    const int t = o / ROWS, row = o % ROWS;
    if (t >= P.T) break;
    const int i = row >> 5, l = (row & 31) + 32 * ((t >> 2) & 1), v = 4 * (t >> 3) + (t & 3);
    float sum = red[(i * 8 + v) * 64 + l];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) sum += red[((w * 2 + i) * 8 + v) * 64 + l];
    const int64_t n = n0 + row;
    if (P.nsplit == 1) P.Y[t * P.N + n] = f32_to_bf16_bits(sum);
    else P.part[((int64_t)z * P.T + t) * P.N + n] = sum;
  }
}

// Y = bf16(sum over slices of the partials), slices added in order.
__global__ __launch_bounds__(256) void k_decode_reduce(const float* __restrict__ part, int nsplit, int64_t total,
                                                       uint16_t* __restrict__ Y) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  float sum = part[idx];
  for (int z = 1; z < nsplit; ++z) sum += part[(int64_t)z * total + idx];
  Y[idx] = f32_to_bf16_bits(sum);
}

}  // namespace

// Contraction slices for an N x K weight: about 448 workgroups, whole stages
// per slice, at most 3 * 256 + SB blocks per slice (so a row touches at most
// MAXG groups of 256 blocks inside one slice).
int decode_splits(int64_t N, int64_t K) {
  const int64_t tiles = N / ROWS;
  const int64_t nbk = K / 64;
  const int64_t nst = (nbk + SB - 1) / SB;
  int64_t ns = (448 + tiles - 1) / tiles;
  if (ns > nst) ns = nst;
  const int64_t min_ns = (nbk + 3 * 256 - 1) / (3 * 256);
  if (ns < min_ns) ns = min_ns;
  return (int)(ns < 1 ? 1 : ns);
}

hipError_t launch_decode(const uint8_t* packed, const uint8_t* codes, const float* consts, const uint16_t* X,
                         int64_t T, int64_t N, int64_t K, const uint16_t* Us, int64_t ldh, const uint16_t* B,
                         int r, int nsplit, float* part, uint16_t* Y, hipStream_t stream) {
  DecodeParams P;
  P.packed = packed; P.codes = codes; P.consts = consts; P.X = X;
  P.T = T; P.N = N; P.K = K;
  P.Us = Us; P.ldh = ldh; P.B = B; P.r = r;
  P.nsplit = nsplit;
  const int64_t nst = (K / 64 + SB - 1) / SB;
  P.per = (nst + nsplit - 1) / nsplit * SB;
  P.Y = Y; P.part = part;
  const Nf4Table& tab = nf4_table();
  for (int i = 0; i < 16; ++i) P.level[i] = tab.level[i];
  const dim3 grid((unsigned)(N / ROWS), (unsigned)nsplit);
  {
    TraceScope ts(KID_DECODE, stream);
    const bool c4 = (K / 64) % 4 == 0;
    if (T <= 4) {
      if (c4) hipLaunchKernelGGL((k_decode<true, 1, 3>), grid, dim3(256), 0, stream, P);
      else hipLaunchKernelGGL((k_decode<false, 1, 3>), grid, dim3(256), 0, stream, P);
    } else if (T <= 8) {
      if (c4) hipLaunchKernelGGL((k_decode<true, 2, 3>), grid, dim3(256), 0, stream, P);
      else hipLaunchKernelGGL((k_decode<false, 2, 3>), grid, dim3(256), 0, stream, P);
    } else {
      if (c4) hipLaunchKernelGGL((k_decode<true, 4, 2>), grid, dim3(256), 0, stream, P);
      else hipLaunchKernelGGL((k_decode<false, 4, 2>), grid, dim3(256), 0, stream, P);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  const int64_t total = T * N;
  TraceScope ts(KID_DECODE_EPILOGUE, stream);
  hipLaunchKernelGGL(k_decode_reduce, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, part, nsplit,
                     total, Y);
  return hipGetLastError();
}

}  // namespace qlora
