// Streaming kernels for the rank-r adapter products of a layer that sees many
// tokens in one call:
//   rows:  C[m][j] = sum_c P[m][c] Qop[j][c]   U = X A^T, G = dY B   ([T][r])
//   cols:  C[m][j] = sum_t P[t][m] Q[t][j]     dA, dB over the hi/lo pairs
// ("QLoRA技术从入门到精通" §3(2)-(3); "LoRA 与 QLoRA：..." §2: the adapter
// branch is B (A x) scaled by alpha / r; only A and B receive gradients.)
//
// Each product reads one large bf16 matrix (X or dY, T x d) exactly once and is
// bound by HBM.  A workgroup owns a block of outputs for one range of the
// contraction (rows) or of the tokens (cols); where a block's range is split
// over several workgroups so that they fill the CUs, the fp32 partial sums go
// to workspace and a second launch adds them in a fixed order, so results are
// deterministic.  What keeps HBM busy is the number of bytes in flight per CU:
// each wave keeps several chunks loading (LDS copies) while it multiplies an
// earlier one.  Rows or contraction positions past the end are read through
// buffer resources with an offset beyond the range, which returns zeros (also
// for copies into LDS).
//
// MFMA v_mfma_f32_16x16x32_bf16.  Fragment layout: lane l holds row (or
// column) l % 16 and contraction slots 8(l/16) .. +7.
#include <algorithm>

#include "dma.hpp"
#include "lora_stream.hpp"
#include "trace.hpp"

namespace qlora {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
using dma::lds_void_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) uint16_t lds_u16_t;

using dma::copy16;
using dma::kOob;
using dma::rsrc;
using dma::v4i_t;
using dma::wait_lds;
using dma::wait_vm;

// MFMA fragment from a row-major LDS tile [rows][ld] whose rows run along the
// contraction: lane l (i = l % 16) receives rows kb .. kb+7 of column c0 + i.
// ds_read_b64_tr_b16: within a 16-lane group, source lane s points at row
// kb + s/4, columns c0 + 4(s%4), and lane i receives rows kb..kb+3 of column c0+i.
__device__ __forceinline__ bf16x8_t tr_frag(const uint16_t* tile, int ld, int kb, int c0) {
  const int s = threadIdx.x & 15;
  const lds_u16_t* base = (const lds_u16_t*)tile;
  const int col = c0 + 4 * (s & 3);
  const int row = kb + (s >> 2);
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(base + row * ld + col));
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(base + (row + 4) * ld + col));
  const u16x8_t v = {(uint16_t)lo[0], (uint16_t)lo[1], (uint16_t)lo[2], (uint16_t)lo[3],
                     (uint16_t)hi[0], (uint16_t)hi[1], (uint16_t)hi[2], (uint16_t)hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// Row-major tiles read with transposing reads: the 16-byte piece p of row R
// is stored at piece p ^ tr_swz(R, pieces per row).  A transposing read (16
// lanes: four rows from a multiple of four, two adjacent pieces; the lanes of
// a 32-lane half take rows 8 further on) then touches each LDS bank at most
// once per 32 lanes (64 banks) and per 16 lanes (32 banks); with an
// unswizzled row of 64 bytes or more those rows fall on the same banks.  Row
// bit 2 is left out, so rows R and R + 4 (the two halves of a fragment) share
// the swizzle.  Widths of other piece counts keep the plain layout.
__device__ __forceinline__ int tr_swz(int row, int ppr) {
  const int b0 = row & 1, b1 = (row >> 1) & 1, b3 = (row >> 3) & 1;
  if (ppr == 4) return 2 * (b1 ^ b3);
  if (ppr == 8) return (2 * b0) ^ (4 * b1) ^ (2 * b3);
  if (ppr == 16 || ppr == 32 || ppr == 64) return (2 * b0) ^ (4 * b1) ^ (8 * b3);
  return 0;
}

// tr_frag from a tile stored with tr_swz (ld elements per row, a multiple of 8)
__device__ __forceinline__ bf16x8_t tr_frag_swz(const uint16_t* tile, int ld, int kb, int c0) {
  const int s = threadIdx.x & 15;
  const lds_u16_t* base = (const lds_u16_t*)tile;
  const int col = c0 + 4 * (s & 3);
  const int row = kb + (s >> 2);
  const int pcol = (((col >> 3) ^ tr_swz(row, ld >> 3)) << 3) | (col & 7);
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(base + row * ld + pcol));
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(base + (row + 4) * ld + pcol));
  const u16x8_t v = {(uint16_t)lo[0], (uint16_t)lo[1], (uint16_t)lo[2], (uint16_t)lo[3],
                     (uint16_t)hi[0], (uint16_t)hi[1], (uint16_t)hi[2], (uint16_t)hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ f32x4_t mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// rows: C[m][j] = sum_c P[m][c] Qop[j][c], m < M, j < r
//
// A workgroup owns 64 rows m for one range of the contraction; the ranges of a
// row tile are split over workgroups so that the row tiles times the ranges
// fill the CUs, and their fp32 partial sums are added in a fixed order by
// k_lora_rows_sum (a single range: the kernel writes the result itself).  Its
// four waves take the range's 64-wide contraction chunks in turn (wave w:
// chunks w, w+4, ...), two in flight each, and add their tiles in LDS in a
// fixed order at the end.  Each chunk's P tile (64 rows x 128 B, from HBM) and
// Q tile (r rows of A x 128 B, or B's contiguous [64][r] block, from L2) are
// copied into the wave's LDS stage: as many bytes of Q as of P, where a tile
// of 16 rows had read four times more of Q than of P.  Contraction-contiguous
// tiles keep whole 128-byte rows; the sixteen-byte piece p of row R sits at
// slot p ^ (R & 7) ^ ((R >> 3) & 1), so a fragment read (16 lanes: 16 rows, one
// piece) touches 16 distinct bank groups.  B's block is read with transposing
// LDS reads.
// ---------------------------------------------------------------------------

constexpr int kRowsChunk = 64;
constexpr int kRowsRT = 64;  // rows per workgroup
constexpr int kRowsPD = 2;   // chunks in flight per wave

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// ROWS/8 copies of a contraction-contiguous tile of ROWS rows (row R at src
// offset base + R * ld * 2 bytes, rows >= valid read as zero) into LDS tile dst
template <int ROWS>
__device__ __forceinline__ void copy_rows(v4i_t rs, uint32_t base, int64_t ld, int valid, uint32_t dst) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < ROWS / 8; ++q) {
    const int R = 8 * q + (lane >> 3);
    const int piece = (lane & 7) ^ swz(R);
    const uint32_t voff = R < valid && base != kOob ? base + (uint32_t)(R * ld * 2 + piece * 16) : kOob;
    copy16(rs, voff, dst + q * 1024);
  }
}

struct RowsLaunch {
  RowsParams p;
  float* part;               // nsplit > 1: [nsplit][M][r] fp32 partial sums
  int32_t nsplit;            // contraction ranges per row tile
  int32_t chunks_per_split;  // 64-wide chunks per range
};

// The final values of row m, column c < ldh of the hi/lo output (and of U
// and the hi/lo pair of the given U), from the row's sum v(j) over j < r.
template <typename SumJ>
__device__ __forceinline__ void rows_out(const RowsParams& p, int64_t m, int c, SumJ v_of) {
  const int r = p.r;
  const int64_t ldh = p.ldh;
  uint16_t h = 0;
  if (c < 2 * r) {
    const int j = c < r ? c : c - r;
    const float v = v_of(j);
    if (p.Vout && c < r) p.Vout[m * r + j] = v;
    uint16_t hi, lo;
    split_bf16(p.s * v, hi, lo);
    h = c < r ? hi : lo;
  }
  p.Hout[m * ldh + c] = h;
  if (p.Ucs) {
    uint16_t u = 0;
    if (c < 2 * r) {
      uint16_t hi, lo;
      split_bf16(p.s * p.Uc[m * r + (c < r ? c : c - r)], hi, lo);
      u = c < r ? hi : lo;
    }
    p.Ucs[m * ldh + c] = u;
  }
}

template <int JT, bool QS>
__global__ __launch_bounds__(256) void k_lora_rows(RowsLaunch L) {
  constexpr int RT = kRowsRT, PD = kRowsPD;
  constexpr int QROWS = 16 * JT;                            // Q tile rows (A) or 64 rows x r (B)
  constexpr int STAGE = RT * 64 + QROWS * 64 + 64;          // bf16 elements (+ slack for transposed reads)
  constexpr int LDR = 16 * JT + 4;                          // row of a wave's tile in the sum, in floats
  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * PD * STAGE];
  static_assert(4 * RT * LDR * 4 <= 4 * PD * STAGE * 2, "the waves' tiles fit over the stages");
  float* red = reinterpret_cast<float*>(lds);               // [wave][RT][LDR], after the loop
  const RowsParams& p = L.p;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int i = lane & 15, g = lane >> 4;
  const int tile = (int)blockIdx.x / L.nsplit, split = (int)blockIdx.x - tile * L.nsplit;
  const int64_t m0 = (int64_t)tile * RT;
  const int64_t nch = p.D / kRowsChunk;
  const int64_t cbeg = (int64_t)split * L.chunks_per_split;
  const int64_t cend = cbeg + L.chunks_per_split < nch ? cbeg + L.chunks_per_split : nch;
  const int64_t mine = cend - cbeg;
  const int nmine = mine > wave ? (int)((mine - wave + 3) / 4) : 0;
  const int iters = (nmine + PD - 1) / PD * PD;
  const int r = p.r;
  // copies per chunk: RT/8 for P, 2JT for Q (copies past r read zeros)
  constexpr int NC = RT / 8 + 2 * JT;

  const v4i_t rp = rsrc(p.P, p.M * p.ldp * 2);
  const v4i_t rq = rsrc(p.Q, QS ? p.D * r * 2 : r * p.ldq * 2);
  const int prows = (int)(p.M - m0 < RT ? p.M - m0 : RT);
  const uint32_t pbase = (uint32_t)(m0 * p.ldp * 2);
  uint16_t* stage0 = lds + wave * PD * STAGE;
  const uint32_t lstage0 = LDS_ADDR(lds) + (uint32_t)(wave * PD * STAGE * 2);

  auto issue = [&](int sp, int k) {
    const int64_t ch = cbeg + wave + 4 * (int64_t)k;
    const bool in = ch < cend;
    const int64_t c0 = ch * kRowsChunk;
    const uint32_t st = lstage0 + (uint32_t)(sp * STAGE * 2);
    copy_rows<RT>(rp, in ? pbase + (uint32_t)(c0 * 2) : kOob, p.ldp, prows, st);
    if (QS) {
      // [64][r] block of B: flat bytes c0*r*2 .. +128r
#pragma unroll
      for (int q = 0; q < 2 * JT; ++q)
        copy16(rq, in && q * 1024 < 128 * r ? (uint32_t)(c0 * r * 2 + q * 1024 + lane * 16) : kOob,
               st + RT * 128 + q * 1024);
    } else {
      copy_rows<QROWS>(rq, in ? (uint32_t)(c0 * 2) : kOob, p.ldq, r, st + RT * 128);
    }
  };

  f32x4_t acc[RT / 16][JT];
#pragma unroll
  for (int rt = 0; rt < RT / 16; ++rt)
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) acc[rt][jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int sp = 0; sp < PD; ++sp) issue(sp, sp);
  for (int k = 0; k < iters; k += PD) {
#pragma unroll
    for (int sp = 0; sp < PD; ++sp) {
      wait_vm<(PD - 1) * NC>();  // this chunk's copies have landed (later chunks issued NC each)
      const uint16_t* st = stage0 + sp * STAGE;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int piece = 4 * ks + g;
        bf16x8_t a[RT / 16];
#pragma unroll
        for (int rt = 0; rt < RT / 16; ++rt) {
          const int prow = 16 * rt + i;
          a[rt] = *reinterpret_cast<const bf16x8_t*>(st + prow * 64 + ((piece ^ swz(prow)) * 8));
        }
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          bf16x8_t b;
          if (QS) {
            b = tr_frag(st + RT * 64, r, 32 * ks + 8 * g, 16 * jt);
          } else {
            const int j = 16 * jt + i < r ? 16 * jt + i : r - 1;
            b = *reinterpret_cast<const bf16x8_t*>(st + RT * 64 + j * 64 + ((piece ^ swz(j)) * 8));
          }
#pragma unroll
          for (int rt = 0; rt < RT / 16; ++rt) acc[rt][jt] = mfma(a[rt], b, acc[rt][jt]);
        }
      }
      wait_lds();  // the stage is read before it is refilled
      issue(sp, k + sp + PD);
    }
  }
  wait_vm<0>();
  __syncthreads();  // every wave is done with the stages the tiles go over

  // fixed-order sum of the four waves' tiles: lane l, value v holds row
  // 16 rt + 4(l/16) + v, column 16 jt + l % 16
#pragma unroll
  for (int rt = 0; rt < RT / 16; ++rt)
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[(wave * RT + 16 * rt + 4 * g + v) * LDR + 16 * jt + i] = acc[rt][jt][v];
  __syncthreads();
  auto sum = [&](int rr, int j) {
    return ((red[(0 * RT + rr) * LDR + j] + red[(1 * RT + rr) * LDR + j]) + red[(2 * RT + rr) * LDR + j]) +
           red[(3 * RT + rr) * LDR + j];
  };
  if (L.nsplit == 1) {
    const int ldh = (int)p.ldh;
    for (int e = threadIdx.x; e < RT * ldh; e += 256) {
      const int rr = e / ldh, c = e % ldh;
      const int64_t m = m0 + rr;
      if (m < p.M) rows_out(p, m, c, [&](int j) { return sum(rr, j); });
    }
  } else {
    float* part = L.part + (int64_t)split * p.M * r;
    for (int e = threadIdx.x; e < RT * r; e += 256) {
      const int rr = e / r, j = e % r;
      const int64_t m = m0 + rr;
      if (m < p.M) part[m * r + j] = sum(rr, j);
    }
  }
}

// The ranges' partial sums, added in range order, then the same outputs as a
// single range writes; thread e takes row e / (r/4 + z), four consecutive
// columns j (16-byte loads of the partials and of U), or one of the z threads
// that clear four padding columns of the hi/lo rows past 2r.
__global__ __launch_bounds__(256) void k_lora_rows_sum(RowsLaunch L) {
  const RowsParams& p = L.p;
  const int r = p.r;
  const int64_t ldh = p.ldh;
  const int q4 = r / 4, z = (int)((ldh - 2 * r) / 4), per = q4 + z;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= p.M * per) return;
  const int64_t m = e / per;
  const int t = (int)(e - m * per);
  if (t >= q4) {  // padding columns 2r + 4(t - q4) .. +3
    const int64_t c = 2 * r + 4 * (t - q4);
    *reinterpret_cast<uint2*>(p.Hout + m * ldh + c) = make_uint2(0u, 0u);
    if (p.Ucs) *reinterpret_cast<uint2*>(p.Ucs + m * ldh + c) = make_uint2(0u, 0u);
    return;
  }
  const int j = 4 * t;
  float4 v = *reinterpret_cast<const float4*>(L.part + m * r + j);
  for (int q = 1; q < L.nsplit; ++q) {
    const float4 w = *reinterpret_cast<const float4*>(L.part + ((int64_t)q * p.M + m) * r + j);
    v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
  }
  if (p.Vout) *reinterpret_cast<float4*>(p.Vout + m * r + j) = v;
  auto pair = [&](float4 a, uint16_t* dst) {
    uint16_t h[4], l[4];
    split_bf16(p.s * a.x, h[0], l[0]);
    split_bf16(p.s * a.y, h[1], l[1]);
    split_bf16(p.s * a.z, h[2], l[2]);
    split_bf16(p.s * a.w, h[3], l[3]);
    *reinterpret_cast<uint2*>(dst + m * ldh + j) =
        make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
    *reinterpret_cast<uint2*>(dst + m * ldh + r + j) =
        make_uint2(l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16));
  };
  pair(v, p.Hout);
  if (p.Ucs) pair(*reinterpret_cast<const float4*>(p.Uc + m * r + j), p.Ucs);
}

// ---------------------------------------------------------------------------
// cols: out[m][j] = sum_t P[t][m] (Q[t][j] + Q[t][j + r]): dA and dB over the
// hi/lo columns of s*G or s*U.
//
// A workgroup of sixteen waves owns 512 output columns m (wave w: columns
// 32w .. 32w+31) for one range of tokens.  The token ranges of a column slab
// are split over workgroups so that every CU has one; their fp32 partial sums
// are added in a fixed order by k_lora_cols_sum (a single range: the kernel
// writes the result itself).  The waves share each 32-token chunk:
// - its P tile [32 t][512 m]: one contiguous kilobyte of each token row, from
//   HBM; pieces of 1 KB per row stream at 5-6 TB/s where pieces of 512 B
//   reached 3.3 TB/s;
// - its Q tile [32 t][128 j]: from L2 (the hi/lo columns are small and every
//   workgroup reads them), staged once per 512 columns of P.
// Four 40 KB stages fill the LDS; one barrier per chunk tells the waves that
// every copy of the chunk has landed and that every wave is done with the
// stage the next copies refill.  Both MFMA operands are read with transposing
// LDS reads (their contraction runs down the rows); the tiles are stored with
// tr_swz, the global piece each lane copies being chosen so that it lands at
// its swizzled place.  The Q tile always holds 128 columns (columns past 2r,
// and tokens past T, only meet outputs that are never stored).  The pair sums
// j + (j + r) are formed in registers: the C fragment of
// v_mfma_f32_16x16x32_bf16 gives lane l column 16 jt + l % 16, so column
// j + r is in the same lane when 16 divides r, else in lane l ^ 8.
// ---------------------------------------------------------------------------

constexpr int kColsWaves = 16;
constexpr int kColsM = 32 * kColsWaves;        // output columns per workgroup
constexpr int kColsJ = 128;                    // staged Q columns (2r <= 128)
constexpr int kColsPD = 4;                     // stages
constexpr int kColsPBytes = 32 * kColsM * 2;   // 32 KB
constexpr int kColsQBytes = 32 * kColsJ * 2;   // 8 KB
constexpr int kColsStage = kColsPBytes + kColsQBytes;
constexpr int kColsCopies = 3;                 // per wave and chunk: two P rows, half a KB of Q

struct ColsLaunch {
  ColsBatch B;
  float* part;            // [split] x (the output's layout) fp32 partial sums of product p at part + part_off[p]
  int64_t part_off[2];
  int32_t nsplit;         // token ranges per column slab
  int32_t chunks_per_split;
  int32_t first_wg[3];    // product p: workgroups first_wg[p] .. first_wg[p+1]-1
};

typedef const __attribute__((address_space(4))) ColsLaunch* ColsLaunchK;

// R: the rank (8 .. 64, a multiple of 8)
template <int R>
__global__ __launch_bounds__(kColsWaves * 64) void k_lora_cols(ColsLaunch L) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kColsPD * kColsStage];
  // the product is a wave-uniform choice; its fields are read in place from the
  // kernel-argument segment (indexing the parameter copy at a run-time index
  // would move it to scratch)
  const ColsLaunchK LK = (ColsLaunchK)__builtin_amdgcn_kernarg_segment_ptr();
  const int pi = (int)blockIdx.x >= L.first_wg[1] && L.B.n > 1 ? 1 : 0;
  const uint16_t* Pp = LK->B.p[pi].P;
  const int64_t ldp = LK->B.p[pi].ldp, D = LK->B.p[pi].D, T = LK->B.p[pi].T;
  const uint16_t* Qp = LK->B.p[pi].Q;
  const int64_t ldq = LK->B.p[pi].ldq;
  const int local = (int)blockIdx.x - (pi ? L.first_wg[1] : 0);
  const int slab = local / L.nsplit, split = local - slab * L.nsplit;
  const int64_t m0 = (int64_t)slab * kColsM;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int g = lane >> 4, i16 = lane & 15;
  const int64_t nch_all = (T + 31) / 32;
  const int64_t c_begin = (int64_t)split * L.chunks_per_split;
  const int64_t c_end = c_begin + L.chunks_per_split < nch_all ? c_begin + L.chunks_per_split : nch_all;
  const int nch = (int)(c_end - c_begin);

  const v4i_t rp = rsrc(Pp, T * ldp * 2);
  const v4i_t rq = rsrc(Qp, T * ldq * 2);
  const uint32_t lds0 = LDS_ADDR(lds);
  // this wave's copies of a chunk: P tile rows wave and wave + 16 (lane l:
  // the row's piece l at its swizzled place), and half a kilobyte of the Q
  // tile, its rows 2 wave and 2 wave + 1 (lanes 0..31)
  uint32_t pv[2];
  bool pin[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int row = wave + kColsWaves * c;
    const int piece = lane ^ tr_swz(row, 64);
    const int64_t col = m0 + 8 * piece;
    pin[c] = col < D;
    pv[c] = (uint32_t)((int64_t)row * ldp * 2 + col * 2);
  }
  const int qrow = 2 * wave + (lane >> 4);
  const uint32_t qv = (uint32_t)((int64_t)qrow * ldq * 2 + (((lane & 15) ^ tr_swz(qrow, 16)) * 16));
  auto issue = [&](int k) {
    const int64_t ch = c_begin + k;
    const bool in = k < nch;
    const uint32_t st = lds0 + (uint32_t)((k % kColsPD) * kColsStage);
    const uint32_t pbase = (uint32_t)(ch * 32 * ldp * 2), qbase = (uint32_t)(ch * 32 * ldq * 2);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = wave + kColsWaves * c;
      copy16(rp, in && pin[c] && ch * 32 + row < T ? pbase + pv[c] : kOob, st + (uint32_t)(row * 1024));
    }
    if (lane < 32) copy16(rq, in && ch * 32 + qrow < T ? qbase + qv : kOob, st + kColsPBytes + (uint32_t)(wave * 512));
  };

  f32x4_t acc[2][8];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) acc[a][jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int k = 0; k < kColsPD - 1; ++k) issue(k);
  for (int k = 0; k < nch; ++k) {
    // chunk k's copies (this wave's) have landed: the later ones in flight are
    // those of chunks k+1 .. k+PD-2
    wait_vm<(kColsPD - 2) * kColsCopies>();
    __syncthreads();  // every wave's copies of chunk k have landed; every wave is done with chunk k-1
    issue(k + kColsPD - 1);  // into the stage of chunk k-1
    const uint16_t* st = reinterpret_cast<const uint16_t*>(lds + (k % kColsPD) * kColsStage);
    bf16x8_t pa[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) pa[a] = tr_frag_swz(st, kColsM, 8 * g, 32 * wave + 16 * a);
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
      const bf16x8_t qb = tr_frag_swz(st + kColsPBytes / 2, kColsJ, 8 * g, 16 * jt);
#pragma unroll
      for (int a = 0; a < 2; ++a) acc[a][jt] = mfma(pa[a], qb, acc[a][jt]);
    }
  }
  wait_vm<0>();

  // lane l holds C[m][j] for m = 32 wave + 16 a + 4 g + v, j = 16 jt + l % 16
  const bool tr = LK->B.p[pi].transposed_out != 0;
  const bool accum = L.nsplit == 1 && LK->B.p[pi].accumulate != 0;
  float* out = L.nsplit > 1 ? L.part + (pi ? L.part_off[1] : L.part_off[0]) + (int64_t)split * D * R
                            : LK->B.p[pi].Fout;
  constexpr int Q16 = R / 16;  // j + r = 16 (jt + Q16) + l % 16 (+ 8 when 16 does not divide R)
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int64_t mb = m0 + 32 * wave + 16 * a + 4 * g;  // m of v = 0
#pragma unroll
    for (int jt = 0; jt < (R + 15) / 16; ++jt) {
      const int j = 16 * jt + i16;
      float t[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float pair;
        if (R % 16 == 0) {
          pair = acc[a][jt + Q16][v];
        } else {
          // column j + r sits in lane l ^ 8: of tile jt + Q16 for l % 16 < 8, of the next one otherwise
          const float send = i16 >= 8 ? acc[a][jt + Q16][v] : acc[a][(jt + Q16 + 1) & 7][v];
          pair = __shfl_xor(send, 8, 16);
        }
        t[v] = acc[a][jt][v] + pair;
      }
      if (j >= R || mb >= D) continue;
      if (tr) {
        // out[j][m .. m+3]: four consecutive m in one 16-byte store
        float4* dst = reinterpret_cast<float4*>(out + (int64_t)j * D + mb);
        float4 o = make_float4(t[0], t[1], t[2], t[3]);
        if (accum) {
          const float4 w = *dst;
          o = make_float4(w.x + o.x, w.y + o.y, w.z + o.z, w.w + o.w);
        }
        *dst = o;
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float* dst = out + (mb + v) * R + j;
          *dst = accum ? *dst + t[v] : t[v];
        }
      }
    }
  }
}

// out = sum over the token ranges, in order, of the partials (+ old out);
// the partials are laid out as the output, so this is a plain stream of
// four-element pieces (D * r is a multiple of 8)
__global__ __launch_bounds__(256) void k_lora_cols_sum(ColsLaunch L) {
  const ColsLaunchK LK = (ColsLaunchK)__builtin_amdgcn_kernarg_segment_ptr();
  const int pi = (int)blockIdx.y;
  if (pi >= L.B.n) return;
  const int64_t n = LK->B.p[pi].D * L.B.p[0].r;
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= n) return;
  const float* part = L.part + (pi ? L.part_off[1] : L.part_off[0]);
  float4 t = *reinterpret_cast<const float4*>(part + e);
  for (int s = 1; s < L.nsplit; ++s) {
    const float4 v = *reinterpret_cast<const float4*>(part + (int64_t)s * n + e);
    t.x += v.x; t.y += v.y; t.z += v.z; t.w += v.w;
  }
  float4* dst = reinterpret_cast<float4*>(LK->B.p[pi].Fout + e);
  if (LK->B.p[pi].accumulate) {
    const float4 o = *dst;
    t.x = o.x + t.x; t.y = o.y + t.y; t.z = o.z + t.z; t.w = o.w + t.w;
  }
  *dst = t;
}

// ---------------------------------------------------------------------------
// U = X A^T for a few tokens (T <= 16), in one launch: workgroup (j, g) owns
// column j of U for the tokens TT*g .. TT*g + TT - 1.  Its 1024 threads walk
// the contraction in pieces of eight (thread t: pieces t, t + 1024, ...), each
// piece one 16-byte load of A's row j and of each of its tokens' X rows, with
// fp32 products; the threads' sums are added in a fixed order (wave shuffles,
// then the 16 waves in LDS).  The workgroup then writes U[t][j], the hi/lo
// pair of s*U[t][j] into Us (columns j and r + j), and its share of Us's zero
// padding.  The tokens per workgroup (TT) are the fewest that keep the grid
// within one workgroup per CU, so that each CU reads A's row and as few X
// rows as the grid allows: with r = 64, one token per workgroup up to four
// tokens, four at sixteen (each workgroup reads 5 rows of K instead of 17).
// ---------------------------------------------------------------------------

constexpr int kSmallDownThreads = 1024;

template <int TT>
__global__ __launch_bounds__(kSmallDownThreads) void k_lora_down_small(SmallDownParams p) {
  constexpr int NW = kSmallDownThreads / 64;
  __shared__ float red[NW][TT];
  const int j = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = (int)blockIdx.y * TT;
  const int T = (int)p.T - t0 < TT ? (int)p.T - t0 : TT;  // this workgroup's tokens, at least one
  const uint16_t* X = p.X + (int64_t)t0 * p.K;
  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = 0.0f;
  const uint16_t* arow = p.A + (int64_t)j * p.K;
  for (int64_t k = (int64_t)tid * 8; k < p.K; k += kSmallDownThreads * 8) {
    // every load of the piece goes out before the first product: token rows
    // t >= T read row T - 1 again, and their sums are never stored
    const uint4 a = *reinterpret_cast<const uint4*>(arow + k);
    uint4 x[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) x[t] = *reinterpret_cast<const uint4*>(X + (int64_t)(t < T ? t : T - 1) * p.K + k);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const uint32_t xw[4] = {x[t].x, x[t].y, x[t].z, x[t].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[t] = fmaf(bf16_bits_to_f32(aw[q] & 0xFFFFu), bf16_bits_to_f32(xw[q] & 0xFFFFu), acc[t]);
        acc[t] = fmaf(bf16_bits_to_f32(aw[q] >> 16), bf16_bits_to_f32(xw[q] >> 16), acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    float v = acc[t];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) red[wave][t] = v;
  }
  __syncthreads();
  if (tid < T) {
    float u = red[0][tid];
#pragma unroll
    for (int w = 1; w < NW; ++w) u += red[w][tid];
    const int64_t t = t0 + tid;
    if (p.U) p.U[t * p.r + j] = u;
    uint16_t hi, lo;
    split_bf16(p.s * u, hi, lo);
    p.Us[t * p.ldh + j] = hi;
    p.Us[t * p.ldh + p.r + j] = lo;
    for (int64_t c = 2 * p.r + j; c < p.ldh; c += p.r) p.Us[t * p.ldh + c] = 0;
  }
}

template <bool QS>
void rows_by_jt(const RowsLaunch& L, int jt, dim3 grid, hipStream_t st, const KernelEvents& ev) {
  const hipEvent_t e0 = ev.start(), e1 = ev.stop();
  switch (jt) {
    case 1: hipExtLaunchKernelGGL((k_lora_rows<1, QS>), grid, dim3(256), 0, st, e0, e1, 0, L); break;
    case 2: hipExtLaunchKernelGGL((k_lora_rows<2, QS>), grid, dim3(256), 0, st, e0, e1, 0, L); break;
    case 3: hipExtLaunchKernelGGL((k_lora_rows<3, QS>), grid, dim3(256), 0, st, e0, e1, 0, L); break;
    default: hipExtLaunchKernelGGL((k_lora_rows<4, QS>), grid, dim3(256), 0, st, e0, e1, 0, L); break;
  }
}

// contraction ranges per row tile: as many workgroups as fill the 256 CUs
// once, each range at least 32 chunks (eight per wave)
int rows_splits(int64_t M, int64_t D) {
  const int64_t tiles = (M + kRowsRT - 1) / kRowsRT;
  int64_t s = 256 / tiles;
  const int64_t cap = D / kRowsChunk / 32;
  if (s > cap) s = cap;
  return (int)(s < 1 ? 1 : s);
}

}  // namespace

bool lora_down_small_ok(int64_t T, int64_t K, int r) { return T >= 1 && T <= 16 && r >= 1 && K % 8 == 0; }

hipError_t launch_lora_down_small(const SmallDownParams& p, hipStream_t stream, int kernel_id) {
  if (!lora_down_small_ok(p.T, p.K, p.r) || p.ldh < 2 * p.r) return hipErrorInvalidValue;
  if (p.T * p.K * 2 > 0x7FFFFFF0LL || (int64_t)p.r * p.K * 2 > 0x7FFFFFF0LL) return hipErrorInvalidValue;
  KernelEvents ev(kernel_id);
  const hipEvent_t e0 = ev.start(), e1 = ev.stop();
  // tokens per workgroup: the fewest that keep r * ceil(T / tt) within 256
  // workgroups, and no more than T rounded up to a power of two
  int tt = 1;
  while (tt < p.T && (int64_t)p.r * ((p.T + tt - 1) / tt) > 256) tt *= 2;
  const dim3 grid((unsigned)p.r, (unsigned)((p.T + tt - 1) / tt));
  const dim3 block(kSmallDownThreads);
  switch (tt) {
    case 1: hipExtLaunchKernelGGL(k_lora_down_small<1>, grid, block, 0, stream, e0, e1, 0, p); break;
    case 2: hipExtLaunchKernelGGL(k_lora_down_small<2>, grid, block, 0, stream, e0, e1, 0, p); break;
    case 4: hipExtLaunchKernelGGL(k_lora_down_small<4>, grid, block, 0, stream, e0, e1, 0, p); break;
    case 8: hipExtLaunchKernelGGL(k_lora_down_small<8>, grid, block, 0, stream, e0, e1, 0, p); break;
    default: hipExtLaunchKernelGGL(k_lora_down_small<16>, grid, block, 0, stream, e0, e1, 0, p); break;
  }
  return hipGetLastError();
}

bool lora_stream_ok(int r) { return r > 0 && r <= 64 && r % 8 == 0; }

// many tokens: at least 512 (r <= 32) or 1024 rows; fewer take the skinny kernel
bool lora_rows_ok(int64_t M, int r) { return lora_stream_ok(r) && M >= (r <= 32 ? 512 : 1024); }

size_t lora_rows_part_bytes(int64_t M, int64_t D, int r) {
  const int s = rows_splits(M, D);
  return s > 1 ? (size_t)s * M * r * 4 : 0;
}

hipError_t launch_lora_rows(const RowsParams& p, float* part, size_t part_bytes, hipStream_t stream, int kernel_id) {
  if (!lora_rows_ok(p.M, p.r) || p.D % 64 != 0 || p.ldh < 2 * p.r || (p.q_strided && p.ldq != p.r))
    return hipErrorInvalidValue;
  if (p.M * p.ldp * 2 > 0x7FFFFFF0LL || (p.q_strided ? p.D * p.r * 2 : p.r * p.ldq * 2) > 0x7FFFFFF0LL)
    return hipErrorInvalidValue;
  RowsLaunch L;
  L.p = p;
  L.nsplit = rows_splits(p.M, p.D);
  if (L.nsplit > 1 && (part == nullptr || part_bytes < lora_rows_part_bytes(p.M, p.D, p.r))) return hipErrorInvalidValue;
  L.part = part;
  const int64_t nch = p.D / kRowsChunk;
  L.chunks_per_split = (int32_t)((nch + L.nsplit - 1) / L.nsplit);
  const int jt = (p.r + 15) / 16;
  const dim3 grid((unsigned)(((p.M + kRowsRT - 1) / kRowsRT) * L.nsplit));
  KernelEvents ev(kernel_id);
  if (p.q_strided) rows_by_jt<true>(L, jt, grid, stream, ev);
  else rows_by_jt<false>(L, jt, grid, stream, ev);
  if (L.nsplit > 1) {
    KernelEvents es(KID_REDUCE);
    const int64_t per = p.r / 4 + (p.ldh - 2 * p.r) / 4;
    const dim3 sg((unsigned)((p.M * per + 255) / 256));
    hipExtLaunchKernelGGL(k_lora_rows_sum, sg, dim3(256), 0, stream, es.start(), es.stop(), 0, L);
  }
  return hipGetLastError();
}

namespace {
// token ranges per column slab: as many workgroups as fit on the 256 CUs in
// one round (one workgroup fills a CU's LDS), each range at least eight chunks
int cols_splits(int64_t T, int64_t slabs) {
  const int64_t nch = (T + 31) / 32;
  int64_t s = 256 / slabs;
  const int64_t cap = nch / 8 > 1 ? nch / 8 : 1;
  if (s > cap) s = cap;
  if (s > 16) s = 16;
  return (int)(s < 1 ? 1 : s);
}
int64_t cols_slabs(int64_t D) { return (D + kColsM - 1) / kColsM; }
}  // namespace

size_t lora_cols_part_bytes(int64_t T, const int64_t* D, int n, int r) {
  int64_t slabs = 0, elems = 0;
  for (int k = 0; k < n; ++k) slabs += cols_slabs(D[k]);
  const int s = cols_splits(T, slabs);
  if (s <= 1) return 0;
  for (int k = 0; k < n; ++k) elems += (int64_t)s * D[k] * r;
  return (size_t)elems * 4;
}

hipError_t launch_lora_cols(const ColsBatch& B, float* part, size_t part_bytes, hipStream_t stream, int kernel_id) {
  if (B.n < 1 || B.n > 2) return hipErrorInvalidValue;
  int64_t slabs = 0, D[2] = {0, 0};
  for (int k = 0; k < B.n; ++k) {
    const ColsParams& p = B.p[k];
    if (p.r != B.p[0].r || p.T != B.p[0].T || !lora_stream_ok(p.r) || p.D % 8 != 0 || p.ldq < 2 * p.r ||
        p.ldp % 8 != 0 || p.ldq % 8 != 0)
      return hipErrorInvalidValue;
    if (p.T * p.ldp * 2 > 0x7FFFFFF0LL || p.T * p.ldq * 2 > 0x7FFFFFF0LL) return hipErrorInvalidValue;
    D[k] = p.D;
    slabs += cols_slabs(p.D);
  }
  ColsLaunch L{};
  L.B = B;
  L.nsplit = cols_splits(B.p[0].T, slabs);
  const int64_t nch = (B.p[0].T + 31) / 32;
  L.chunks_per_split = (int32_t)((nch + L.nsplit - 1) / L.nsplit);
  if (L.nsplit > 1) {
    if (!part || part_bytes < lora_cols_part_bytes(B.p[0].T, D, B.n, B.p[0].r)) return hipErrorInvalidValue;
    L.part = part;
    L.part_off[0] = 0;
    L.part_off[1] = (int64_t)L.nsplit * D[0] * B.p[0].r;
  }
  L.first_wg[0] = 0;
  for (int k = 0; k < B.n; ++k) L.first_wg[k + 1] = L.first_wg[k] + (int32_t)(cols_slabs(D[k]) * L.nsplit);
  for (int k = B.n; k < 2; ++k) L.first_wg[k + 1] = L.first_wg[k];
  {
    KernelEvents ev(kernel_id);
    const dim3 grid((unsigned)L.first_wg[B.n]), block(kColsWaves * 64);
    const hipEvent_t e0 = ev.start(), e1 = ev.stop();
    switch (B.p[0].r) {
      case 8: hipExtLaunchKernelGGL(k_lora_cols<8>, grid, block, 0, stream, e0, e1, 0, L); break;
      case 16: hipExtLaunchKernelGGL(k_lora_cols<16>, grid, block, 0, stream, e0, e1, 0, L); break;
      case 24: hipExtLaunchKernelGGL(k_lora_cols<24>, grid, block, 0, stream, e0, e1, 0, L); break;
      case 32: hipExtLaunchKernelGGL(k_lora_cols<32>, grid, block, 0, stream, e0, e1, 0, L); break;
      case 40: hipExtLaunchKernelGGL(k_lora_cols<40>, grid, block, 0, stream, e0, e1, 0, L); break;
      case 48: hipExtLaunchKernelGGL(k_lora_cols<48>, grid, block, 0, stream, e0, e1, 0, L); break;
      case 56: hipExtLaunchKernelGGL(k_lora_cols<56>, grid, block, 0, stream, e0, e1, 0, L); break;
      default: hipExtLaunchKernelGGL(k_lora_cols<64>, grid, block, 0, stream, e0, e1, 0, L); break;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || L.nsplit <= 1) return e;
  const int64_t dr = std::max(D[0], D[1]) * B.p[0].r;
  KernelEvents ev(KID_REDUCE);
  hipExtLaunchKernelGGL(k_lora_cols_sum, dim3((unsigned)((dr / 4 + 255) / 256), (unsigned)B.n), dim3(256), 0, stream,
                        ev.start(), ev.stop(), 0, L);
  return hipGetLastError();
}

}  // namespace qlora
