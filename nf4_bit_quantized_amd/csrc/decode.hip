// Forward for few tokens (T <= 16): stream the packed weight once.
//
// With at most 16 tokens the product X W_hat^T is bound by reading the packed
// nibbles and scale codes from HBM ("QLoRA技术从入门到精通" §3(2): the 4-bit
// weight is restored block by block at compute time and discarded).
//
// Work split: the rows are cut into 16-row tiles and every workgroup owns a
// run of NTW consecutive tiles over the whole contraction (NTW = N/16/256
// rounded up, so the weight shapes of a transformer give every CU the same
// share and no partial sums leave the workgroup).  The workgroup's DW waves
// split the contraction into chunks of 128 weights (wave w: chunks w, w+DW, ...)
// and add their tiles in LDS in a fixed order at the end.
//
// Loads: per tile, one 16-byte load per lane covers 16 rows x 64 contiguous
// bytes of a chunk; it goes to registers, and is issued again for the wave's
// next chunk as soon as the tile has been restored, so a wave keeps about one
// chunk per tile in flight while it computes.  The chunk's X rows (256 bytes
// each) come densely from L2, one 16-byte load per lane per 4 token rows, and
// reach the MFMA layout through the wave's LDS slot.  The workgroup's scale
// codes (one contiguous run) and the ratios c_g / 255 of their groups are
// copied to LDS once, while the table is built, so the loop reads a chunk's two
// codes with one LDS read.
//
// MFMA v_mfma_f32_16x16x32_bf16, A = X (16 token rows), B = restored weights
// (16 rows): lane l holds row l%16 and contraction slots 8(l/16) .. +7.  One
// MFMA covers half a 64-weight block (32 weights), so the block's two MFMA
// results form the block's own sum, which is multiplied by the row's restored
// scale s' = fl32(code) * fl32(c_g / 255) and added to the fp32 accumulator.
// (This differs from rounding T[q] * s' to bf16 by at most one bf16 rounding
// of each weight.)  The loaded 16 bytes of lane group g are bytes 16g.. of the
// row chunk; a 4 x 4 transpose of the four dwords across the lane groups
// (v_permlane32_swap, v_permlane16_swap) gives group g dword 4j + g for half
// block j, i.e. contraction slots 64(j/2) + 32(j%2) + 8g.
//
// Restore: a packed byte (levels q_hi, q_lo) indexes a 256-entry table of the
// pairs bf16(T[q_hi]), bf16(T[q_lo]) in element order.  Each lane has a private
// copy of the table in its own LDS bank (entry v of lane L at dword 64v + L,
// 64 KB at LDS offset 0), so the 64 lanes of a lookup never conflict, and the
// address (v << 8) | 4L is one v_perm_b32 of the packed dword and 4L.
//
// Rank-r term: added per tile after the sum, s (X A^T) B^T through the same
// MFMA over the 2r hi/lo columns of s U (zero-padded to a multiple of 64).
//
// Without the second level (fp32 block scales, "7、QLoRA 量化微调" §7.1) the
// workgroup's block scales (one contiguous run, 57 KB at the 8192 <-> 28672
// shapes) are copied straight to LDS (buffer loads into LDS, no registers) in
// place of the codes, each row at a stride of sst floats, an odd multiple of
// four, so that 16 rows read at one column (8 bytes each) fall in distinct
// banks; the loop reads a chunk's two scales with one LDS read.
#include "decode.hpp"
#include "dma.hpp"
#include "trace.hpp"

namespace qlora {

namespace {

constexpr int LUT_DWORDS = 256 * 64;      // 64 KB
constexpr int CODES_BYTES = 32 * 1024;    // the workgroup's scale codes and group ratios
constexpr int SCALES_BYTES = 64 * 1024;   // or, without the second level, its fp32 block scales
constexpr uint32_t kOob = 0x80000000u;    // buffer offset past every range used here: loads read zero

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct DecodeParams {
  const uint8_t* packed;
  const uint8_t* codes;
  const float* consts;
  const uint16_t* X;   // [T][K]
  int64_t T, N, K;
  const uint16_t* Us;  // hi/lo pair of s*U, [T][ldh], zero past 2r (unused when r == 0)
  int64_t ldh;
  const uint16_t* B;   // [N][r]
  int r;
  uint16_t* Y;         // [T][N]
  int bshift;          // log2(weights per absmax block / 64); K is a multiple of the block
  float level[16];
  // contraction split: with nsplit > 1 the workgroups of a run of tiles take
  // nsplit consecutive ranges of the chunks and store their sums to
  // part[split][T][N] (the first range's with the rank-r term); k_decode_sum
  // adds them and rounds Y
  int nsplit;
  float* part;
};

// Several weights that share X (the projections of one layer input) in one
// launch: workgroups first_wg[i] .. first_wg[i+1]-1 take the row tiles of
// weight i.  T, K and the block format are the same for all of them.
constexpr int kMaxProj = kDecodeMaxWeights;
struct DecodeMulti {
  DecodeParams p[kMaxProj];
  int first_wg[kMaxProj + 1];
  int n;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int64_t bytes) {
  const int32_t n = bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0 : (int32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}

// One chunk's loads of one wave: X (XQ loads of 4 token rows x 256 bytes) and
// the packed 16 bytes of each tile.
template <int NTW, int XQ>
struct ChunkRegs {
  u32x4_t x[XQ];
  u32x4_t w[NTW];
};

// Four table lookups of the bytes of packed dword d -> 8 restored bf16 in element order.
__device__ __forceinline__ bf16x8_t lookup8(uint32_t d, uint32_t lanebase) {
  typedef __attribute__((address_space(3))) const uint32_t lds_cu32_t;
  u32x4_t o;
  o.x = *reinterpret_cast<lds_cu32_t*>((uintptr_t)__builtin_amdgcn_perm(d, lanebase, 0x0C0C0400u));
  o.y = *reinterpret_cast<lds_cu32_t*>((uintptr_t)__builtin_amdgcn_perm(d, lanebase, 0x0C0C0500u));
  o.z = *reinterpret_cast<lds_cu32_t*>((uintptr_t)__builtin_amdgcn_perm(d, lanebase, 0x0C0C0600u));
  o.w = *reinterpret_cast<lds_cu32_t*>((uintptr_t)__builtin_amdgcn_perm(d, lanebase, 0x0C0C0700u));
  return __builtin_bit_cast(bf16x8_t, o);
}

// 4 x 4 transpose of dwords across the four 16-lane groups: afterwards group
// g's register j holds what group j's register g held.
__device__ __forceinline__ void transpose4(uint32_t& a, uint32_t& b, uint32_t& c, uint32_t& d) {
  const auto p = __builtin_amdgcn_permlane32_swap(a, c, false, false);
  const auto q = __builtin_amdgcn_permlane32_swap(b, d, false, false);
  const auto s = __builtin_amdgcn_permlane16_swap(p[0], q[0], false, false);
  const auto t = __builtin_amdgcn_permlane16_swap(p[1], q[1], false, false);
  a = s[0]; b = s[1]; c = t[0]; d = t[1];
}

__device__ __forceinline__ f32x4_t mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// DW: waves per workgroup (8 or 16).  NTW: 16-row tiles per workgroup.  XQ: X
// loads per chunk (1 for T <= 4, else 4).  CODES2: K/64 is even, so a chunk's
// two codes are one aligned 2-byte LDS read and its two blocks (an even block
// index and the next) never straddle a group of 256 blocks.  F32S: fp32 block
// scales in consts (no codes).
template <int DW, int NTW, int XQ, bool CODES2, bool F32S = false>
__global__ __launch_bounds__(DW * 64) void k_decode(DecodeMulti M) {
  // this workgroup's weight (a wave-uniform choice)
  int pi = 0;
  for (int q = 1; q < M.n; ++q) pi += (int)blockIdx.x >= M.first_wg[q] ? 1 : 0;
  const DecodeParams& P = M.p[pi];
  constexpr int DT = DW * 64;
  // chunks in flight per wave besides the reissued tiles (registers: 128 per
  // lane with 16 waves, 256 with 8)
  constexpr int PD = DW == 16 ? (NTW <= 2 ? 2 : 1) : (NTW <= 2 ? 3 : (NTW <= 5 ? 2 : 1));
  constexpr int XSW = XQ * 1024;          // a wave's X slot: 4 XQ token rows x 256 bytes
  constexpr int RED = 8 * NTW * 1024;     // eight waves' partial tiles, after the loop
  constexpr int AUXB = F32S ? SCALES_BYTES : CODES_BYTES;  // the staged scales
  constexpr int REGION = AUXB + DW * XSW > RED ? AUXB + DW * XSW : RED;
  // the table must sit at LDS offset 0 (its addresses are formed without a base):
  // this is the kernel's only LDS variable
  __shared__ __attribute__((aligned(16))) uint32_t lds[LUT_DWORDS + REGION / 4];
  uint32_t* lut = lds;
  uint8_t* aux = reinterpret_cast<uint8_t*>(lds + LUT_DWORDS);
  float* red = reinterpret_cast<float*>(aux);  // [wave][tile][v][lane]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, g = lane >> 4;
  const uint32_t lanebase = (uint32_t)lane * 4u;
  // every byte offset below fits 32 bits: the packed weight is below 2 GiB
  const int T = (int)P.T, K = (int)P.K;
  const int ntiles = (int)(P.N / 16);
  const int local = (int)blockIdx.x - M.first_wg[pi];
  const int split = local % P.nsplit;
  const int nt0 = local / P.nsplit * NTW;
  const int nbk = K / 64;             // 64-weight halves of chunks per row
  const int nbc = nbk >> P.bshift;    // scale codes (or fp32 scales) per row
  const int sst = 4 * (((nbc + 3) >> 2) | 1);  // LDS row stride of the fp32 scales, in floats
  // this workgroup's chunks c_lo .. c_hi - 1 (all of them without a split)
  const int nch_all = (K + 127) / 128;
  const int cps = (nch_all + P.nsplit - 1) / P.nsplit;
  const int c_lo = split * cps;
  const int c_hi = c_lo + cps < nch_all ? c_lo + cps : nch_all;
  const int nch = c_hi - c_lo;
  const int nmine = nch > wave ? (nch - wave + DW - 1) / DW : 0;
  const int iters = (nmine + PD - 1) / PD * PD;

  const __amdgpu_buffer_rsrc_t rw = rsrc(P.packed, P.N * P.K / 2);
  const __amdgpu_buffer_rsrc_t rx = rsrc(P.X, P.T * P.K * 2);
  const __amdgpu_buffer_rsrc_t rc = rsrc(P.codes, F32S ? 0 : P.N * nbc);
  const __amdgpu_buffer_rsrc_t rk = rsrc(P.consts, F32S ? P.N * nbc * 4 : ((P.N * nbc + 255) / 256) * 4);

  // the workgroup's codes: rows nt0*16 .. are one contiguous, 16-byte aligned
  // run of 16*NTW*nbc bytes in memory (rows past N read zero); in LDS each row
  // starts at a multiple of rs bytes, rs/4 odd, so that 16 consecutive rows
  // read at one column fall in distinct banks.  Then the ratios c_g / 255 of
  // the groups of 256 blocks the run spans.  Without the second level the run
  // is the rows' fp32 scales, 64*NTW*nbc bytes, and there are no ratios.
  const uint32_t cfirst = (uint32_t)nt0 * 16u * (uint32_t)nbc;
  const uint32_t cbytes = (F32S ? 64u : 16u) * NTW * (uint32_t)nbc;
  const uint32_t rs = 4u * (((uint32_t)(nbc + 3) >> 2) | 1u);
  const uint32_t g_lo = cfirst >> 8;
  const uint32_t ngr = F32S ? 0u : ((cfirst + cbytes - 1u) >> 8) - g_lo + 1u;
  float* ratio = reinterpret_cast<float*>(aux + ((16u * NTW * rs + 15u) & ~15u));
  constexpr int CQ = F32S ? 0 : AUXB / 16 / DT;
  u32x4_t cv[CQ > 0 ? CQ : 1];
#pragma unroll
  for (int q = 0; q < CQ; ++q) {
    const uint32_t o = (uint32_t)(tid + q * DT) * 16u;
    cv[q] = __builtin_amdgcn_raw_buffer_load_b128(rc, o < cbytes ? cfirst + o : kOob, 0, 0);
  }
  if (F32S) {
    // the scales' LDS image in 16-byte slots: row j's slot p holds its scales
    // 4p .. 4p+3 (slots past the row's scales read zero, or the next row's
    // first scales, never used); copy c of the workgroup fills slots
    // 64c .. 64c+63, wave w issuing copies w, w + DW, ...
    const dma::v4i_t rd = dma::rsrc(P.consts, P.N * nbc * 4);
    const uint32_t spr = (uint32_t)sst / 4u, nslots = 16u * NTW * spr, pieces = ((uint32_t)nbc + 3u) / 4u;
#pragma unroll
    for (int c = 0; c < 64 / DW; ++c) {
      const uint32_t cc = (uint32_t)(wave + DW * c);
      if (64u * cc < nslots) {
        const uint32_t slot = 64u * cc + (uint32_t)lane, row = slot / spr, p = slot - row * spr;
        const uint32_t src = (cfirst + row * (uint32_t)nbc + 4u * p) * 4u;
        dma::copy16(rd, slot < nslots && p < pieces ? src : kOob, LDS_ADDR(aux) + 1024u * cc);
      }
    }
  }
  // (no load at all without the second level, so that exactly the chunk loads
  // below follow the scale copies)
  const float cg = F32S ? 0.f
                        : __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                        rk, (uint32_t)tid < ngr ? (g_lo + (uint32_t)tid) * 4u : kOob, 0, 0));

  // this lane's row of tile i is n0 + 16 i
  const uint32_t n0 = (uint32_t)nt0 * 16u + (uint32_t)i16;
  const uint32_t wbase = n0 * (uint32_t)(K / 2) + 16u * (uint32_t)g;  // packed byte of tile 0, chunk 0
  const uint32_t wtile = 16u * (uint32_t)(K / 2);                      // packed bytes per tile
  // X load q: lane l holds piece l%16 (16 bytes) of token row 4q + l/16 of the chunk
  const int xp = lane & 15;
  const uint32_t xbase = (uint32_t)g * (uint32_t)(K * 2) + 16u * (uint32_t)xp;
  // X slot: piece p of token row t at piece position p ^ t (conflict-free reads);
  // with one load per chunk only rows 0..3 exist, and lanes of rows >= 4 read
  // row i16 % 4 (MFMA rows are independent and token rows >= T are never stored)
  uint8_t* xs = aux + AUXB + wave * XSW;
  const int xrow = XQ == 1 ? (i16 & 3) : i16;

  auto issue_x = [&](ChunkRegs<NTW, XQ>& R, int k) {
    const int ch = c_lo + wave + DW * k;
    const bool in = ch < c_hi && ch * 128 + 8 * xp < K;
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
      const bool tin = in && 4 * q + g < T;
      R.x[q] = __builtin_amdgcn_raw_buffer_load_b128(
          rx, tin ? xbase + (uint32_t)(4 * q) * (uint32_t)(K * 2) + (uint32_t)ch * 256u : kOob, 0, 0);
    }
  };
  auto issue_w = [&](ChunkRegs<NTW, XQ>& R, int i, int k) {
    const int ch = c_lo + wave + DW * k;
    const bool in = ch < c_hi && ch * 64 + 16 * g < K / 2 && nt0 + i < ntiles;
    R.w[i] = __builtin_amdgcn_raw_buffer_load_b128(
        rw, in ? wbase + (uint32_t)i * wtile + (uint32_t)ch * 64u : kOob, 0, 0);
  };

  // the first chunks' loads go out before the table is built
  ChunkRegs<NTW, XQ> R[PD];
#pragma unroll
  for (int sp = 0; sp < PD; ++sp) {
    issue_x(R[sp], sp);
#pragma unroll
    for (int i = 0; i < NTW; ++i) issue_w(R[sp], i, sp);
  }

  // byte table: entry v = (bf16(T[v >> 4]), bf16(T[v & 15])), one copy per
  // lane bank; a wave writes whole entries, so the levels are read with scalar
  // loads (a vector load here would make the waits below drain the loads
  // already in flight)
  for (int v = wave; v < 256; v += DW)
    lut[v * 64 + lane] = pack_bf16x2(P.level[v >> 4], P.level[v & 15]);
#pragma unroll
  for (int q = 0; q < CQ; ++q) {
    const uint32_t o = (uint32_t)(tid + q * DT) * 16u;
    if (o < cbytes) {
      const uint32_t w4[4] = {cv[q].x, cv[q].y, cv[q].z, cv[q].w};
      uint32_t row = o / (uint32_t)nbc, col = o - row * (uint32_t)nbc;
      if ((nbc & 3) == 0) {  // dwords never straddle rows
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          *reinterpret_cast<uint32_t*>(aux + row * rs + col) = w4[d];
          col += 4u;
          if (col >= (uint32_t)nbc) { col -= (uint32_t)nbc; ++row; }
        }
      } else {
#pragma unroll
        for (int b = 0; b < 16; ++b) {
          aux[row * rs + col] = (uint8_t)(w4[b >> 2] >> (8 * (b & 3)));
          if (++col == (uint32_t)nbc) { col = 0u; ++row; }
        }
      }
    }
  }
  if ((uint32_t)tid < ngr) ratio[tid] = restored_scale(1u, cg);  // fl32(c_g / 255)

  f32x4_t acc[NTW];
#pragma unroll
  for (int i = 0; i < NTW; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // this wave's scale copies have landed: only the first chunks' loads (XQ + NTW
  // per chunk), issued after them, may still be in flight
  if (F32S) dma::wait_vm<PD * (XQ + NTW)>();
  __syncthreads();  // the table, codes and ratios (or scales) are in place

  for (int k = 0; k < iters; k += PD) {
#pragma unroll
    for (int sp = 0; sp < PD; ++sp) {
      const int ch = c_lo + wave + DW * (k + sp);
      const bool chin = ch < c_hi;
      const int chc = chin ? ch : 0;
      // X through the wave's slot into the MFMA layout; the slot's reads of the
      // previous chunk precede these writes in the wave's LDS order
#pragma unroll
      for (int q = 0; q < XQ; ++q) {
        const int t = 4 * q + g;
        *reinterpret_cast<u32x4_t*>(xs + t * 256 + ((xp ^ t) & 15) * 16) = R[sp].x[q];
      }
      bf16x8_t xa[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xa[j] = *reinterpret_cast<const bf16x8_t*>(xs + xrow * 256 + (((4 * j + g) ^ xrow) & 15) * 16);
      issue_x(R[sp], k + sp + PD);
#pragma unroll
      for (int i = 0; i < NTW; ++i) {
        uint32_t d0 = R[sp].w[i].x, d1 = R[sp].w[i].y, d2 = R[sp].w[i].z, d3 = R[sp].w[i].w;
        transpose4(d0, d1, d2, d3);  // dj: half block j of this lane group
        // s' = fl32(code) * fl32(c_g / 255) of the chunk's two blocks of this
        // lane's row (zero for a chunk past the row's end, whose weights read zero)
        const uint32_t row = (uint32_t)(16 * i + i16);
        float s0, s1;
        if (F32S) {
          // the chunk's two halves' scales: blocks 2ch and 2ch + 1 (64 weights),
          // or one block for both (blocks of 128 or 256); one aligned 8-byte read
          const uint32_t b0 = (uint32_t)(2 * chc) >> P.bshift;
          const float2 v = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(aux) +
                                                            row * (uint32_t)sst + (b0 & ~1u));
          const float lo = (b0 & 1u) ? v.y : v.x;
          s0 = lo;
          s1 = 2 * chc + 1 < nbk ? (P.bshift == 0 ? v.y : lo) : 0.f;
        } else if (CODES2) {  // 64-weight blocks, an even count per row
          const uint32_t cl = row * rs + (uint32_t)(2 * chc);                     // code byte in LDS
          const uint32_t gb = cfirst + row * (uint32_t)nbc + (uint32_t)(2 * chc);  // its block index
          const uint32_t c2 = *reinterpret_cast<const uint16_t*>(aux + cl);
          const float rt = ratio[(gb >> 8) - g_lo];
          s0 = (float)(c2 & 0xFFu) * rt;
          s1 = (float)(c2 >> 8) * rt;
        } else {  // the two halves' blocks (one and the same when blocks hold 128 or 256 weights)
          const bool two = 2 * chc + 1 < nbk;
          const uint32_t b0 = (uint32_t)(2 * chc) >> P.bshift, b1 = (uint32_t)(2 * chc + 1) >> P.bshift;
          const uint32_t gb0 = cfirst + row * (uint32_t)nbc + b0, gb1 = cfirst + row * (uint32_t)nbc + b1;
          s0 = (float)aux[row * rs + b0] * ratio[(gb0 >> 8) - g_lo];
          s1 = two ? (float)aux[row * rs + b1] * ratio[(gb1 >> 8) - g_lo] : 0.f;
        }
        s0 = chin ? s0 : 0.f;
        s1 = chin ? s1 : 0.f;
        f32x4_t c = mfma(xa[0], lookup8(d0, lanebase), f32x4_t{0.f, 0.f, 0.f, 0.f});
        c = mfma(xa[1], lookup8(d1, lanebase), c);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][v] = fmaf(s0, c[v], acc[i][v]);
        c = mfma(xa[2], lookup8(d2, lanebase), f32x4_t{0.f, 0.f, 0.f, 0.f});
        c = mfma(xa[3], lookup8(d3, lanebase), c);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][v] = fmaf(s1, c[v], acc[i][v]);
        // the tile's next load, into the registers just consumed (issued once
        // they are free, so the loop carries no register copies, which would
        // wait for the load), and kept here by the scheduling barriers
        __builtin_amdgcn_sched_barrier(0);
        issue_w(R[sp], i, k + sp + PD);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // wave w < NTW finishes tile w; its rank-r operands are fetched before the
  // partial tiles are added (r a multiple of 8 and 2r <= 128: A = hi/lo
  // columns of s U, token rows >= T read zero; B = B[n][j % r])
  const bool fin = wave < NTW && nt0 + wave < ntiles;
  const int64_t n = (int64_t)n0 + 16 * wave;
  const bool tok = i16 < T;
  constexpr int MJ = 4;
  const bool tail = split == 0;  // the first range carries the rank-r term
  const bool pre = tail && P.r > 0 && (P.r & 7) == 0 && P.ldh <= 32 * MJ;
  const __amdgpu_buffer_rsrc_t ru = rsrc(P.Us, P.T * P.ldh * 2);
  u32x4_t ua[MJ], ub[MJ];
  if (fin && pre) {
#pragma unroll
    for (int q = 0; q < MJ; ++q) {
      if (32 * q < P.ldh) {
        ua[q] = __builtin_amdgcn_raw_buffer_load_b128(
            ru, tok ? (uint32_t)((i16 * P.ldh + 32 * q + 8 * g) * 2) : kOob, 0, 0);
        ub[q] = *reinterpret_cast<const u32x4_t*>(P.B + n * P.r + (32 * q + 8 * g) % P.r);
      }
    }
  }

  // add the waves' tiles in a fixed order: (w + (w + 8)) for w < 8, then
  // w = 0 .. 7; lane l, value v holds token 4(l/16) + v of row l%16
  __syncthreads();  // every wave is done with the codes and its X slot
  if (DW == 16 && wave >= 8) {
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[(((wave - 8) * NTW + i) * 4 + v) * 64 + lane] = acc[i][v];
  }
  if (DW == 16) __syncthreads();
  if (wave < 8) {
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float* r = &red[((wave * NTW + i) * 4 + v) * 64 + lane];
        *r = DW == 16 ? acc[i][v] + *r : acc[i][v];
      }
  }
  __syncthreads();
  if (!fin) return;
  f32x4_t c;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float sum = red[((0 * NTW + wave) * 4 + v) * 64 + lane];
#pragma unroll
    for (int w = 1; w < 8; ++w) sum += red[((w * NTW + wave) * 4 + v) * 64 + lane];
    c[v] = sum;
  }
  if (pre) {
#pragma unroll
    for (int q = 0; q < MJ; ++q)
      if (32 * q < P.ldh) c = mfma(__builtin_bit_cast(bf16x8_t, ua[q]), __builtin_bit_cast(bf16x8_t, ub[q]), c);
  } else if (tail && P.r > 0) {
    for (int64_t jj = 0; jj < P.ldh; jj += 32) {
      const uint32_t uo = tok ? (uint32_t)((i16 * P.ldh + jj + 8 * g) * 2) : kOob;
      const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(ru, uo, 0, 0);
      const uint32_t j0 = (uint32_t)((jj + 8 * g) % P.r);
      uint16_t e[8];
      for (int q = 0; q < 8; ++q) e[q] = P.B[n * P.r + (j0 + q) % (uint32_t)P.r];
      const u32x4_t b = {e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16), e[4] | ((uint32_t)e[5] << 16),
                         e[6] | ((uint32_t)e[7] << 16)};
      c = mfma(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c);
    }
  }
  if (P.nsplit > 1) {  // this range's sum; k_decode_sum adds the ranges and rounds
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = 4 * g + v;
      if (t < T) P.part[((int64_t)split * T + t) * P.N + n] = c[v];
    }
    return;
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int t = 4 * g + v;
    if (t < T) P.Y[t * P.N + n] = f32_to_bf16_bits(c[v]);
  }
}

// Y = bf16(part[0] + part[1] + ...) after a split launch, the ranges added in
// range order; four consecutive outputs per thread (N is a multiple of 16).
__global__ __launch_bounds__(256) void k_decode_sum(DecodeParams P) {
  const int64_t tn = P.T * P.N;
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;  // t * N + n
  if (e >= tn) return;
  float4 v = *reinterpret_cast<const float4*>(P.part + e);
  for (int q = 1; q < P.nsplit; ++q) {
    const float4 w = *reinterpret_cast<const float4*>(P.part + q * tn + e);
    v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
  }
  const uint2 y = {(uint32_t)f32_to_bf16_bits(v.x) | ((uint32_t)f32_to_bf16_bits(v.y) << 16),
                   (uint32_t)f32_to_bf16_bits(v.z) | ((uint32_t)f32_to_bf16_bits(v.w) << 16)};
  *reinterpret_cast<uint2*>(P.Y + e) = y;
}

// 16 waves where their 128 registers per lane hold the loop, else 8
template <int NTW>
void launch_ntw(const DecodeMulti& P, bool c2, bool f32s, unsigned grid, hipStream_t stream) {
  const dim3 g(grid);
  KernelEvents ev(KID_DECODE);
  const hipEvent_t e0 = ev.start(), e1 = ev.stop();
  if (f32s) {  // 16 waves' X slots for 16 tokens and the staged scales would overflow LDS
    if (P.p[0].T <= 4) {
      if constexpr (NTW <= 7)
        hipExtLaunchKernelGGL((k_decode<16, NTW, 1, false, true>), g, dim3(1024), 0, stream, e0, e1, 0, P);
      else hipExtLaunchKernelGGL((k_decode<8, NTW, 1, false, true>), g, dim3(512), 0, stream, e0, e1, 0, P);
    } else {
      hipExtLaunchKernelGGL((k_decode<8, NTW, 4, false, true>), g, dim3(512), 0, stream, e0, e1, 0, P);
    }
  } else if (c2 && P.p[0].T <= 4) {
    if constexpr (NTW <= 7) hipExtLaunchKernelGGL((k_decode<16, NTW, 1, true>), g, dim3(1024), 0, stream, e0, e1, 0, P);
    else hipExtLaunchKernelGGL((k_decode<8, NTW, 1, true>), g, dim3(512), 0, stream, e0, e1, 0, P);
  } else if (c2) {
    if constexpr (NTW <= 6) hipExtLaunchKernelGGL((k_decode<16, NTW, 4, true>), g, dim3(1024), 0, stream, e0, e1, 0, P);
    else hipExtLaunchKernelGGL((k_decode<8, NTW, 4, true>), g, dim3(512), 0, stream, e0, e1, 0, P);
  } else if (P.p[0].T <= 4) {
    hipExtLaunchKernelGGL((k_decode<8, NTW, 1, false>), g, dim3(512), 0, stream, e0, e1, 0, P);
  } else {
    hipExtLaunchKernelGGL((k_decode<8, NTW, 4, false>), g, dim3(512), 0, stream, e0, e1, 0, P);
  }
}

}  // namespace

// LDS bytes of the fp32 scales of t 16-row tiles (rows at stride sst floats).
static int64_t f32_scales_bytes(int64_t K, int bshift, int64_t t) {
  const int64_t nbc = (K / 64) >> bshift;
  return 64 * t * 4 * (((nbc + 3) / 4) | 1);
}

// Rows hold whole blocks, and the workgroup's codes (or fp32 scales) must fit
// their LDS region with at least one 16-row tile.
bool decode_supported(int64_t N, int64_t K, int bshift, bool f32s) {
  if (N % 16 != 0 || K % (64 << bshift) != 0 || N * K / 2 > 0x7FFFFFF0LL) return false;
  if (f32s) return N * ((K / 64) >> bshift) * 4 <= 0x7FFFFFF0LL && f32_scales_bytes(K, bshift, 1) <= SCALES_BYTES;
  const int64_t nbc = (K / 64) >> bshift;
  const int64_t rs = 4 * (((nbc + 3) / 4) | 1);
  return ((16 * rs + 15) & ~15LL) + 4 * (16 * nbc / 256 + 2) <= CODES_BYTES;
}

// Tiles per workgroup for weights of ntiles_all 16-row tiles in all: spread
// over the 256 CUs (at most 8 each), then cut until the workgroup's codes and
// group ratios (or fp32 scales) fit their LDS region.  0: nothing fits.
static int64_t decode_ntw(int64_t ntiles_all, int64_t K, int bshift, bool f32s) {
  int64_t ntw = (ntiles_all + 255) / 256;
  if (ntw > 8) ntw = 8;
  const int64_t nbc = (K / 64) >> bshift;             // scale codes per row
  const int64_t rs = 4 * (((nbc + 3) / 4) | 1);      // LDS row stride of the codes
  auto aux_need = [&](int64_t t) { return ((16 * t * rs + 15) & ~15LL) + 4 * (16 * t * nbc / 256 + 2); };
  while (!f32s && ntw > 1 && aux_need(ntw) > CODES_BYTES) --ntw;
  if (!f32s && aux_need(ntw) > CODES_BYTES) return 0;
  while (f32s && ntw > 1 && f32_scales_bytes(K, bshift, ntw) > SCALES_BYTES) --ntw;
  if (f32s && f32_scales_bytes(K, bshift, ntw) > SCALES_BYTES) return 0;
  return ntw;
}

// More than four tokens on a weight of at most 512 tiles: X (T rows of 256
// bytes per chunk) outweighs the workgroup's one or two tiles of packed bytes
// (1 KB each per chunk).  Two workgroups per run of twice the tiles, each over
// half the contraction, halve the X each reads; their sums go through
// part[2][T][N] and k_decode_sum.  Codes only (the fp32 scales of twice the
// tiles would overflow LDS), and at least 64 chunks so that each of the 16
// waves keeps two.
int decode_split(int64_t T, int64_t N, int64_t K, int bshift, bool f32s) {
  if (f32s || T <= 4 || T > 16 || !decode_supported(N, K, bshift, f32s) || (K + 127) / 128 < 64) return 1;
  const int64_t ntw = decode_ntw(N / 16, K, bshift, f32s);
  if (ntw < 1 || ntw > 2) return 1;
  return decode_ntw(2 * ntw * 256, K, bshift, f32s) == 2 * ntw ? 2 : 1;
}

size_t decode_part_bytes(int64_t T, int64_t N, int64_t K, int bshift, bool f32s) {
  const int sp = decode_split(T, N, K, bshift, f32s);
  return sp > 1 ? (size_t)sp * T * N * 4 : 0;
}

static hipError_t decode_launch(const DecodeWeight* w, int n, const uint16_t* X, int64_t T, int64_t K,
                                const uint16_t* const* Us, int64_t ldh, int r, int bshift, bool f32s, int nsplit,
                                float* part, hipStream_t stream) {
  // byte offsets into the packed weight, codes and X are 32-bit
  if (n < 1 || n > kMaxProj || T < 1 || T > 16 || bshift < 0 || bshift > 2) return hipErrorInvalidValue;
  if (nsplit > 1 && (n != 1 || !part)) return hipErrorInvalidValue;
  DecodeMulti M{};
  M.n = n;
  int64_t ntiles_all = 0;
  for (int i = 0; i < n; ++i) {
    if (!decode_supported(w[i].N, K, bshift, f32s)) return hipErrorInvalidValue;
    DecodeParams& P = M.p[i];
    P.packed = w[i].packed; P.codes = w[i].codes; P.consts = w[i].consts; P.X = X;
    P.T = T; P.N = w[i].N; P.K = K;
    P.Us = Us[i]; P.ldh = ldh; P.B = w[i].B; P.r = r;
    P.Y = w[i].Y;
    P.bshift = bshift;
    const Nf4Table& tab = level_table(w[i].table);
    for (int j = 0; j < 16; ++j) P.level[j] = tab.level[j];
    P.nsplit = nsplit;
    P.part = part;
    ntiles_all += w[i].N / 16;
  }
  // with a split, each run of tiles is twice as long and has nsplit workgroups
  const int64_t ntw = decode_ntw(nsplit * ntiles_all, K, bshift, f32s);
  if (ntw < 1) return hipErrorInvalidValue;
  int64_t wg = 0;
  for (int i = 0; i < n; ++i) {
    M.first_wg[i] = (int)wg;
    wg += (w[i].N / 16 + ntw - 1) / ntw * nsplit;
  }
  M.first_wg[n] = (int)wg;
  const unsigned grid = (unsigned)wg;
  const bool c2 = bshift == 0 && (K / 64) % 2 == 0;
  switch (ntw) {
    case 1: launch_ntw<1>(M, c2, f32s, grid, stream); break;
    case 2: launch_ntw<2>(M, c2, f32s, grid, stream); break;
    case 3: launch_ntw<3>(M, c2, f32s, grid, stream); break;
    case 4: launch_ntw<4>(M, c2, f32s, grid, stream); break;
    case 5: launch_ntw<5>(M, c2, f32s, grid, stream); break;
    case 6: launch_ntw<6>(M, c2, f32s, grid, stream); break;
    case 7: launch_ntw<7>(M, c2, f32s, grid, stream); break;
    default: launch_ntw<8>(M, c2, f32s, grid, stream); break;
  }
  if (nsplit > 1) {
    KernelEvents ev(KID_DECODE_SUM);
    hipExtLaunchKernelGGL(k_decode_sum, dim3((unsigned)((T * w[0].N / 4 + 255) / 256)), dim3(256), 0, stream,
                          ev.start(), ev.stop(), 0, M.p[0]);
  }
  return hipGetLastError();
}

hipError_t launch_decode_multi(const DecodeWeight* w, int n, const uint16_t* X, int64_t T, int64_t K,
                               const uint16_t* const* Us, int64_t ldh, int r, int bshift, bool f32s,
                               hipStream_t stream) {
  return decode_launch(w, n, X, T, K, Us, ldh, r, bshift, f32s, 1, nullptr, stream);
}

hipError_t launch_decode(const uint8_t* packed, const uint8_t* codes, const float* consts, const uint16_t* X,
                         int64_t T, int64_t N, int64_t K, const uint16_t* Us, int64_t ldh, const uint16_t* B,
                         int r, uint16_t* Y, int table, int bshift, bool f32s, float* part, size_t part_bytes,
                         hipStream_t stream) {
  const DecodeWeight w{packed, codes, consts, N, B, Y, table};
  int sp = decode_split(T, N, K, bshift, f32s);
  if (sp > 1 && (!part || part_bytes < (size_t)sp * T * N * 4)) sp = 1;
  return decode_launch(&w, 1, X, T, K, &Us, ldh, r, bshift, f32s, sp, part, stream);
}

}  // namespace qlora
