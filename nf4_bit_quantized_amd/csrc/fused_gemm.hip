// The two large products of the layer with the NF4 restore fused in:
//   forward  Y  = bf16( X W_hat^T + [sU_hi | sU_lo] [B | B]^T )
//   backward dX = bf16( dY W_hat  + [sG_hi | sG_lo] [A ; A] )
//
// "QLoRA技术从入门到精通" §3(2) restores the 4-bit weight at compute time
// (table value times the block's stored scale, to a 16-bit float) and
// discards it; "【X 长文】..." (storage and compute paragraph) restores each
// 64-weight block to bf16 just before it enters the product.  Here every
// 64-weight block is restored once per workgroup into an LDS bf16 tile and fed
// to v_mfma_f32_32x32x16_bf16; the restored weight never reaches memory.
//
// Restore without table lookups in LDS: a thread that restores one block first
// builds, in registers, the 16 values bf16(T[i] * s') of that block (16 fp32
// products, 8 pack-converts) split into a high-byte table and a low-byte table
// of four registers each; each 4-bit index is then resolved with v_perm_b32
// byte selects (three per byte table per four indices), so a packed word of 8
// indices costs about 29 VALU instructions and no memory access.  The values
// are exactly bf16_rne(fl32(T[q] * s')).
//
// Tiling (gfx950: 256 CUs, 4 SIMDs each, 160 KB LDS; measured per CU: LDS
// reads ~240 B/clk, global loads ~55 B/clk): 512 threads.  Waves 0-3 multiply
// (2 x 2 grid, wave tile 128 x 64 of 32 x 32 MFMA tiles, workgroup tile
// 256 x 128, contraction step 64); waves 4-7 restore weights.  One barrier per
// step.
//
// The activation operand (X or dY) goes from global memory straight to LDS
// (buffer_load_dwordx4 ... lds): the multiplying waves issue those copies for
// step t+2 between their MFMAs of step t, two per sixteen-wide contraction
// slice, so the per-CU load path (~55 B/clk) is never hit by a burst and no
// VGPR or VALU work is spent on it.  Three A stages (t, t+1 landing, t+2 being
// issued); before the barrier that ends step t each wave waits until its
// copies for step t+1 have landed.  A tiles are 256 rows of 128 B without
// padding; sixteen-byte chunk c of row R sits at position
// c ^ (R & 7) ^ ((R >> 3) & 1), so a fragment read (16 lanes per LDS cycle: 16
// consecutive rows, one chunk) touches 16 distinct 16-byte bank groups.
//
// The restoring waves load the packed words, codes and group constants of step
// t+3 into registers and restore step t+1 into one of two B stages while step t
// is multiplied.  Forward B rows are contraction-contiguous and padded to
// 144 B, which is conflict-free for the same fragment reads.
//
// dX contracts over d_out, the row index of the packed weight.  The restored
// tile is stored row-major ([k][n], rows padded to 288 B) exactly as it comes
// from memory, and the MFMA B fragments (8 consecutive k at one n) are read
// with ds_read_b64_tr_b16: within each 16-lane group, source lane s points at
// row kb + s/4, columns c0 + 4*(s%4), and lane i receives the four rows
// kb..kb+3 of column c0 + i.
//
// The LoRA term runs as extra contraction steps over the 2r columns of a
// hi/lo bf16 split of s*U (forward) or s*G (dX), so it is accumulated in fp32
// with the base product before the single rounding of the output.
//
// Output: the fp32 tile is converted to bf16 into LDS and stored with
// coalesced 16-byte writes.  Workgroups are ordered so that the tiles a single
// XCD (round-robin by workgroup id) works on form a compact block (two tile
// rows), keeping the operands they share in that XCD's L2.
#include <cstdlib>

#include "fused.hpp"
#include "restore.hpp"
#include "trace.hpp"

namespace qlora {
namespace {

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // contraction-contiguous LDS row: 72 bf16 = 144 B


typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

template <int BN, bool BT>
struct Geometry {
  static constexpr int BM = 256;
  static constexpr int TM = 4;              // 32-row MFMA tiles per wave (wave rows 128)
  static constexpr int TN = BN / 64;        // 32-col MFMA tiles per wave
  static constexpr int A_BYTES = BM * BK * 2;  // one A stage: 256 rows of 128 B
  // B tile: [BN][LDK] (contraction-contiguous) or [64][BN] (column-contiguous,
  // swizzled: see bt_col)
  static constexpr int LDB_T = BN;
  static constexpr int B_ELEMS = BT ? BK * LDB_T : BN * LDK;
  static constexpr int B_BYTES = B_ELEMS * 2;
  static constexpr int B_OFF = 3 * A_BYTES;    // the two B stages follow the three A stages
  static constexpr int LDC = BN + 8;           // epilogue bf16 tile row
  static constexpr int MAIN_BYTES = B_OFF + 2 * B_BYTES;
  static constexpr int LDS_BYTES = MAIN_BYTES > BM * LDC * 2 ? MAIN_BYTES : BM * LDC * 2;
};

// Column-contiguous B tile (dX): element (row, col) sits in row `row` at
// column bt_col(row, col).  Columns move in units of four (8 bytes, what one
// lane of a transposed fragment read takes); unit u of row r goes to unit
// u ^ 10 (r mod 4).  With 64 four-byte banks and a 256-byte row, a fragment
// read (32 lanes at a time: four consecutive rows from a multiple of four,
// eight consecutive units from a multiple of eight) and a restore store (16
// lanes at a time: four consecutive rows, 16-byte pieces at units 8q + 2i)
// then each touch every bank once.  Units 2i and 2i + 1 stay adjacent, so a
// 16-byte store stays one store.
__device__ __forceinline__ int bt_col(int row, int col) {
  return (((col >> 2) ^ (10 * (row & 3))) << 2) | (col & 3);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int64_t bytes) {
  const int32_t n = bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0 : (int32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}

// ---------------------------------------------------------------------------
// A operand: global -> LDS copies issued by the multiplying waves
//
// Multiplying wave cw copies rows 64cw .. 64cw+63 of each A stage with eight
// 1 KB copies; copy j covers rows 64cw + 8j .. +7, lane l lands at byte 16l of
// it, i.e. row 64cw + 8j + l/8, position l%8, and so fetches chunk
// (l%8) ^ (l/8) ^ (j%2) of that row (the swizzle above).  Rows beyond the
// output are clamped to the last row: they only feed output rows never stored.
// ---------------------------------------------------------------------------

struct ACopy {
  __amdgpu_buffer_rsrc_t r;
  uint32_t voff[8];  // per-lane byte offsets at contraction column 0
};

__device__ __forceinline__ ACopy make_acopy(const uint16_t* A, int64_t ld, int64_t M, int64_t m0, int cw, int lane) {
  ACopy c;
  c.r = rsrc(A, M * ld * 2);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int64_t row = m0 + 64 * cw + 8 * j + (lane >> 3);
    row = row < M ? row : M - 1;
    const int chunk = (lane & 7) ^ (lane >> 3) ^ (j & 1);
    c.voff[j] = (uint32_t)(row * ld * 2 + chunk * 16);
  }
  return c;
}

// Copy j of this wave's rows for the contraction columns starting at byte col_bytes.
__device__ __forceinline__ void a_copy(const ACopy& c, uint32_t col_bytes, uint8_t* stage, int cw, int j) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(c.r, (lds_void_t*)(stage + (64 * cw + 8 * j) * 128), 16, c.voff[j],
                                           col_bytes, 0, 0);
}

// Wait until at most n of this wave's global loads (here: its A copies) are in flight.
template <int N>
__device__ __forceinline__ void wait_copies() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ---------------------------------------------------------------------------
// Restoring waves: packed words, codes, group constants -> registers (issued
// early), restored bf16 -> LDS
//
// Main-loop loads are buffer loads whose per-thread byte offsets are computed
// once; the contraction step advances through the scalar offset.  Weight
// rows/columns beyond the output are clamped to a valid address instead of
// masked: they only feed output columns that are never stored.
// ---------------------------------------------------------------------------

template <int BN>
struct StepRegs {
  uint32_t w[BN / 32];   // packed weight words (8 indices each)
  uint32_t code4;        // the aligned dword holding the block's 8-bit scale code
  uint32_t code_shift;   // bit position of the code inside code4
  float cg;
};

struct Cursor {
  __amdgpu_buffer_rsrc_t rw, rc, rk;
  uint32_t woff;     // byte offset of the thread's packed words at step 0
  uint32_t coff;     // 64-weight chunk index of the thread's weights at step 0
  uint32_t wstep;    // bytes the packed words advance per step
  uint32_t cstep;    // chunks the chunk index advances per step
  uint32_t nk;       // contraction steps
  uint32_t rot;      // this workgroup starts its contraction at step rot (see fused_body)
  uint32_t bshift;   // 64-weight chunk index >> bshift = absmax block index
  uint32_t dq;       // 1: codes + group constants; 0: fp32 block scales in consts
  uint32_t nseg;     // dX over several weights: their contraction steps follow each other,
  uint32_t k0[kMaxFusedSegs + 1];  // weight i's first (unrotated) step k0[i]
  uint32_t lo, hi;   // several weights: rw, rc, rk are those of the weight with steps [lo, hi)
};

// Buffer resources of one stored weight of `rows` rows: packed words, scale
// codes, group constants (or fp32 block scales).
__device__ __forceinline__ void weight_rsrcs(const FusedParams& P, const uint8_t* packed, const uint8_t* codes,
                                             const float* consts, int64_t rows, Cursor& c) {
  c.rw = rsrc(packed, rows * P.Kw / 2);
  const int64_t nblocks = (rows * P.Kw / 64) >> P.bshift;
  c.rc = rsrc(codes, P.dq ? nblocks : 0);
  c.rk = rsrc(consts, P.dq ? ((nblocks + 255) / 256) * 4 : nblocks * 4);
}

// Restoring-wave thread index: those are waves 4..7 of the workgroup.
__device__ __forceinline__ int ptid() { return (int)threadIdx.x - 256; }

template <int BN, bool BT>
__device__ __forceinline__ void w_coords(int& lrow, int& lcol) {
  const int tid = ptid();
  if (!BT) {
    // forward: BN rows of 64 weights; one row (BN = 256) or half a row (BN = 128) per thread
    if (BN == 256) { lrow = tid; lcol = 0; }
    else { lrow = tid >> 1; lcol = (tid & 1) * 32; }
  } else {
    // dX: 64 rows (contraction) of BN columns; four threads per row
    lrow = tid >> 2;
    lcol = (tid & 3) * (BN / 4);
  }
}

template <int BN, bool BT>
__device__ __forceinline__ Cursor make_cursor(const FusedParams& P, int64_t n0) {
  Cursor c;
  weight_rsrcs(P, P.packed, P.codes, P.consts, BT ? P.K0 : P.N, c);
  c.bshift = (uint32_t)P.bshift;
  c.dq = (uint32_t)P.dq;
  int lrow, lcol;
  w_coords<BN, BT>(lrow, lcol);
  if (!BT) {
    int64_t n = n0 + lrow;
    n = n < P.N ? n : P.N - 1;
    c.woff = (uint32_t)(n * (P.Kw / 2) + lcol / 2);
    c.coff = (uint32_t)(n * (P.Kw / 64));
    c.wstep = BK / 2;
    c.cstep = 1;
  } else {
    int64_t k = n0 + lcol;
    k = (k < P.N ? k : 0) + P.col0;
    c.woff = (uint32_t)(lrow * (P.Kw / 2) + k / 2);
    c.coff = (uint32_t)(lrow * (P.Kw / 64) + k / 64);
    c.wstep = (uint32_t)(BK * (P.Kw / 2));
    c.cstep = (uint32_t)(BK * (P.Kw / 64));
  }
  return c;
}

// contraction step -> stored column block (the workgroup's rotated order)
__device__ __forceinline__ uint32_t rotated(uint32_t step, uint32_t rot, uint32_t nk) {
  const uint32_t kt = step + rot;
  return kt >= nk ? kt - nk : kt;
}

// Several weights: lookups by segment index go through fixed-bound unrolled
// selects on a wave-uniform index, so the parameter block and the k0 table
// stay in scalar registers (an index known only at run time would copy them
// to scratch memory).
__device__ __forceinline__ int seg_of(uint32_t kt, const uint32_t (&k0)[kMaxFusedSegs + 1], int nseg) {
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxFusedSegs; ++i) si = (i < nseg && kt >= k0[i]) ? i : si;
  return __builtin_amdgcn_readfirstlane(si);
}

__device__ __forceinline__ uint32_t k0_of(const uint32_t (&k0)[kMaxFusedSegs + 1], int si) {
  uint32_t v = 0;
#pragma unroll
  for (int i = 1; i <= kMaxFusedSegs; ++i) v = si == i ? k0[i] : v;
  return v;
}

// The kernels' one argument, read in place from the kernel-argument segment
// (it starts there, at offset 0).  A field of segment si, si known only at
// run time but the same for the whole wave, is then one scalar load at a
// computed offset; indexing the by-value parameter itself at a run-time
// index would copy all of it to scratch memory first.
typedef const __attribute__((address_space(4))) FusedParams* KernargParams;

__device__ __forceinline__ KernargParams kernarg_params() {
  return (KernargParams)__builtin_amdgcn_kernarg_segment_ptr();
}

template <int BN>
__device__ __forceinline__ void fetch(StepRegs<BN>& f, Cursor& c, uint32_t step, const FusedParams& P) {
  uint32_t kt = rotated(step, c.rot, c.nk);
  if (c.nseg > 1) {
    // several weights (dX): the step's weight and its step within that weight;
    // the resources change only when the step enters another weight
    if (kt < c.lo || kt >= c.hi) {
      const int si = seg_of(kt, c.k0, (int)c.nseg);
      c.lo = k0_of(c.k0, si);
      c.hi = k0_of(c.k0, si + 1);
      if (si == 0) {
        weight_rsrcs(P, P.packed, P.codes, P.consts, P.K0, c);
      } else {
        const KernargParams K = kernarg_params();
        weight_rsrcs(P, K->seg[si].packed, K->seg[si].codes, K->seg[si].consts, K->seg[si].N, c);
      }
    }
    kt -= c.lo;
  }
  const __amdgpu_buffer_rsrc_t rw = c.rw, rc = c.rc, rk = c.rk;
  const uint32_t sw = kt * c.wstep;
  const u32x4_t w0 = __builtin_amdgcn_raw_buffer_load_b128(rw, c.woff, sw, 0);
  f.w[0] = w0.x; f.w[1] = w0.y; f.w[2] = w0.z; f.w[3] = w0.w;
  if (BN == 256) {
    const u32x4_t w1 = __builtin_amdgcn_raw_buffer_load_b128(rw, c.woff + 16, sw, 0);
    f.w[4] = w1.x; f.w[5] = w1.y; f.w[6] = w1.z; f.w[7] = w1.w;
  }
  const uint32_t blk = (c.coff + kt * c.cstep) >> c.bshift;
  // the codes array holds N*K/blocksize bytes, a multiple of 4, so the aligned dword is in range;
  // without the second level the code load reads zero (empty range) and cg is the block's scale
  f.code4 = __builtin_amdgcn_raw_buffer_load_b32(rc, blk & ~3u, 0, 0);
  f.code_shift = (blk & 3u) * 8u;
  f.cg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rk, (c.dq ? blk >> 8 : blk) * 4, 0, 0));
}

// Keeps the scheduler from hoisting work on prefetched registers above the
// point of use: an early use of a late load would wait for every load issued
// before it (loads complete in order) and drain the prefetch.
template <int BN>
__device__ __forceinline__ void pin(StepRegs<BN>& f) {
  asm volatile("" : "+v"(f.code4), "+v"(f.cg));
#pragma unroll
  for (int i = 0; i < BN / 32; ++i) asm volatile("" : "+v"(f.w[i]));
}

template <int BN, bool BT>
__device__ __forceinline__ void restore_step(StepRegs<BN>& f, const Nf4Table& tab, int dq,
                                             uint16_t* __restrict__ Bs) {
  pin<BN>(f);
  int lrow, lcol;
  w_coords<BN, BT>(lrow, lcol);
  const RestoreTab t = make_tab(tab, dq ? restored_scale((f.code4 >> f.code_shift) & 0xFFu, f.cg) : f.cg);
  static_assert(!BT || BN == 128, "the dX tile swizzle covers 128 columns");
  // dX: the four threads of a row store their 16-byte pieces (8 columns each)
  // in two orders: threads 2 and 3 start with their third piece.  A 16-byte
  // store is done 8 lanes (two rows) at a time on 32 banks, where threads 0
  // and 2 of a row, 64 columns apart, would otherwise share banks; with the
  // tile swizzle (bt_col) every store then touches each bank once.
  const bool rot = BT && (ptid() & 2) != 0;
  const uint32_t w0 = rot ? f.w[2] : f.w[0], w1 = rot ? f.w[3] : f.w[1];
  const uint32_t w2 = rot ? f.w[0] : f.w[2], w3 = rot ? f.w[1] : f.w[3];
  const uint32_t ww[4] = {w0, w1, w2, w3};
  // dX: the restored columns stay in the order 0, 2, 4, 6, 1, 3, 5, 7 inside
  // each group of eight (restore8_evenodd); the rank-r tail's rows are stored
  // in the same order, and the epilogue puts the output columns back
#pragma unroll
  for (int i = 0; i < BN / 32; i += 2) {
    uint32_t o[8];
    if (BT) {
      restore8_evenodd(ww[i], t, o);
      restore8_evenodd(ww[i + 1], t, o + 4);
    } else {
      restore8(f.w[i], t, o);
      restore8(f.w[i + 1], t, o + 4);
    }
    const int c0 = BT ? lcol + (((i + (rot ? 2 : 0)) & 3) * 8) : lcol + i * 8;
    const int c1 = BT ? lcol + (((i + 1 + (rot ? 2 : 0)) & 3) * 8) : lcol + i * 8 + 8;
    uint16_t* d0 = BT ? Bs + lrow * Geometry<BN, BT>::LDB_T + bt_col(lrow, c0) : Bs + lrow * LDK + c0;
    uint16_t* d1 = BT ? Bs + lrow * Geometry<BN, BT>::LDB_T + bt_col(lrow, c1) : Bs + lrow * LDK + c1;
    *reinterpret_cast<uint4*>(d0) = make_uint4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<uint4*>(d1) = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

// LoRA tail B operand (bf16, small): forward Bop[n][kk] = B[n][kk % r],
// dX Bop[kk][k] = A[kk % r][k].  Columns kk >= 2r meet zeros in the tail A
// operand, so they need no masking.  Written straight to LDS.
template <int BN, bool BT>
__device__ __forceinline__ void tail_b_store(const uint16_t* __restrict__ Bt, int64_t ldbt, int r, int64_t cols,
                                             int64_t n0, int64_t kt, uint16_t* __restrict__ Bs) {
  const int tid = ptid();
  if (!BT) {
    for (int c = tid; c < BN * 8; c += 256) {
      const int lrow = c >> 3, kc = (c & 7) * 8;
      int64_t n = n0 + lrow;
      n = n < cols ? n : cols - 1;
      const uint32_t kk = (uint32_t)(kt * BK + kc);
      uint4 v;
      if ((r & 7) == 0) {
        v = *reinterpret_cast<const uint4*>(Bt + n * ldbt + kk % (uint32_t)r);
      } else {
        uint16_t e[8];
        for (int q = 0; q < 8; ++q) e[q] = Bt[n * ldbt + (kk + q) % (uint32_t)r];
        v = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
      }
      *reinterpret_cast<uint4*>(Bs + lrow * LDK + kc) = v;
    }
  } else {
    constexpr int LDB_T = Geometry<BN, BT>::LDB_T;
    for (int c = tid; c < BK * (BN / 8); c += 256) {
      const int lrow = c / (BN / 8), lc = (c % (BN / 8)) * 8;
      const int64_t kk = kt * BK + lrow;
      int64_t col = n0 + lc;
      col = col < cols ? col : 0;
      // the eight columns in the restore's order 0, 2, 4, 6, 1, 3, 5, 7
      const uint4 v = *reinterpret_cast<const uint4*>(Bt + (int64_t)((uint32_t)kk % (uint32_t)r) * ldbt + col);
      *reinterpret_cast<uint4*>(Bs + lrow * LDB_T + bt_col(lrow, lc)) =
          make_uint4(perm(v.y, v.x, 0x05040100u), perm(v.w, v.z, 0x05040100u), perm(v.y, v.x, 0x07060302u),
                     perm(v.w, v.z, 0x07060302u));
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA fragments of one sixteen-wide contraction slice, and their products
// ---------------------------------------------------------------------------

template <int BN>
struct Frags {
  bf16x8_t a[4];
  bf16x8_t b[BN / 64];
};

template <int BN, bool BT>
__device__ __forceinline__ void load_frags(Frags<BN>& f, const uint8_t* __restrict__ As,
                                           const uint16_t* __restrict__ Bs, uint32_t arow, uint32_t apos, int ks) {
  constexpr int TM = 4, TN = BN / 64;
  const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) & 1;
  const int kofs = ks * 16 + (lane >> 5) * 8;
#pragma unroll
  for (int i = 0; i < TM; ++i) f.a[i] = *reinterpret_cast<const bf16x8_t*>(As + arow + i * 4096 + apos);
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    if (!BT) {
      f.b[j] = *reinterpret_cast<const bf16x8_t*>(Bs + ((wn * TN + j) * 32 + (lane & 31)) * LDK + kofs);
    } else {
      constexpr int LDB_T = Geometry<BN, BT>::LDB_T;
      const int s = lane & 15;
      const int col = (wn * TN + j) * 32 + ((lane >> 4) & 1) * 16 + 4 * (s & 3);
      const int row = kofs + (s >> 2);
      typedef __attribute__((address_space(3))) uint16_t lds_u16_t;
      const lds_u16_t* base = (const lds_u16_t*)Bs;
      // rows row and row + 4 share row & 3, so both reads take the same swizzled column
      const int scol = bt_col(row, col);
      const u16x4_t lo = __builtin_bit_cast(
          u16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(base + row * LDB_T + scol)));
      const u16x4_t hi = __builtin_bit_cast(
          u16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(base + (row + 4) * LDB_T + scol)));
      typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
      const u16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      f.b[j] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
}

template <int BN>
__device__ __forceinline__ void mma_frags(const Frags<BN>& f, f32x16_t (&acc)[4][BN / 64]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < BN / 64; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// ---------------------------------------------------------------------------
// The kernel body
// ---------------------------------------------------------------------------

// MULTI: dX over several weights (P.nseg of them); a kernel of its own, so
// the single-weight kernels carry none of the segment code.
template <int BN, bool BT, bool MULTI = false>
__device__ __forceinline__ void fused_body(const FusedParams& P) {
  using G = Geometry<BN, BT>;
  constexpr int TM = G::TM, TN = G::TN;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[G::LDS_BYTES];

  // tile order: chunks of consecutive tiles go to one XCD; inside the order,
  // groups of two tile rows are walked column by column.
  const int64_t ntiles = (int64_t)P.mt * P.nt;
  const int64_t chunk = (ntiles + 7) / 8;
  const int64_t order = (int64_t)(blockIdx.x % 8) * chunk + blockIdx.x / 8;
  if (order >= ntiles) return;
  const int gm = P.group_m;
  const int64_t group = order / ((int64_t)gm * P.nt);
  const int64_t first_m = group * gm;
  const int64_t rows_in_group = (P.mt - first_m) < gm ? (P.mt - first_m) : gm;
  const int64_t in_group = order - group * gm * P.nt;
  const int64_t tm = first_m + in_group % rows_in_group;
  const int64_t tn = in_group / rows_in_group;
  const int64_t m0 = tm * G::BM, n0 = tn * BN;

  // several weights (dX only): main steps of weight 0, 1, ..., then the
  // rank-r tail steps of weight 0, 1, ...
  const int nseg = MULTI ? P.nseg : 1;
  uint32_t k0[kMaxFusedSegs + 1];  // past the last weight every entry is nk
  k0[0] = 0;
  k0[1] = (uint32_t)(P.K0 / BK);
#pragma unroll
  for (int i = 1; i < kMaxFusedSegs; ++i) k0[i + 1] = k0[i] + (i < nseg ? (uint32_t)(P.seg[i].N / BK) : 0u);
  const uint32_t nk = k0[kMaxFusedSegs];
  const uint32_t ntail1 = P.r > 0 ? (uint32_t)((2 * (int64_t)P.r + BK - 1) / BK) : 0;  // per weight
  const uint32_t ntail = ntail1 * nseg;
  const uint32_t nsteps = nk + ntail;
  // Tiles of one tile row share their A rows and walk the contraction in
  // lockstep, so those rows are read once into L2 and hit there.  Different
  // tile rows start at different steps: rows a power of two apart would
  // otherwise send the same column block of every row to few L2 channels
  // at once.  The sum order per tile is fixed, so results stay deterministic.
  const uint32_t rot = (uint32_t)((tm * 5) % nk);
  auto a_stage = [&](uint32_t s) { return lds + (s % 3) * G::A_BYTES; };
  auto b_stage = [&](uint32_t s) { return reinterpret_cast<uint16_t*>(lds + G::B_OFF + (s & 1) * G::B_BYTES); };

  // Both roles pass the same sequence of barriers: 1 + nsteps, then 2.
  if (threadIdx.x < 256) {
    const int lane = threadIdx.x & 63;
    const int cw = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wm = cw >> 1;
    // fragment addresses: row wm*128 + i*32 + lane%32, chunk 2ks + lane/32
    const uint32_t arow = (uint32_t)((wm * 128 + (lane & 31)) * 128);
    const int x = (lane & 7) ^ ((lane >> 3) & 1);
    uint32_t apos[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) apos[ks] = (uint32_t)(((2 * ks + (lane >> 5)) ^ x) * 16);

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // A copies, issued in step order: steps < nk read the rotated column block
    // of X / dY, step nk + t the hi/lo columns 64t .. 64t+63.
    ACopy cp = make_acopy(P.A, P.lda, P.M, m0, cw, lane);
    // the source of step c's copies: key i < kMaxFusedSegs is weight i's
    // activation, kMaxFusedSegs + i its hi/lo tail columns
    auto key_of = [&](uint32_t c) {
      if (c < nk) return seg_of(rotated(c, rot, nk), k0, nseg);
      return __builtin_amdgcn_readfirstlane(kMaxFusedSegs + (int)((c - nk) / ntail1));
    };
    int cp_key = 0;
    auto source_key = [&](int key) {
      if (key != cp_key) {
        cp_key = key;
        const int si = key % kMaxFusedSegs;
        if (key == 0) {
          cp = make_acopy(P.A, P.lda, P.M, m0, cw, lane);
        } else if (key < kMaxFusedSegs) {
          const KernargParams K = kernarg_params();
          cp = make_acopy(K->seg[si].A, K->seg[si].lda, P.M, m0, cw, lane);
        } else if (si == 0) {
          cp = make_acopy(P.At, P.ldat, P.M, m0, cw, lane);
        } else {
          const KernargParams K = kernarg_params();
          cp = make_acopy(K->seg[si].At, K->seg[si].ldat, P.M, m0, cw, lane);
        }
      }
    };
    auto source = [&](uint32_t c) { source_key(key_of(c)); };
    // the source and column of step c < nsteps in one pass, with scalar
    // selects only (several weights; run every step, so no division)
    auto key_col = [&](uint32_t c, int& key, uint32_t& col) {
      const bool tail = c >= nk;
      uint32_t x = tail ? c - nk : rotated(c, rot, nk);
      // (formed in vector registers: the scalar file is full in this loop)
      asm volatile("" : "+v"(x));
      int si = 0;
      uint32_t base = 0;
#pragma unroll
      for (int i = 1; i < kMaxFusedSegs; ++i) {
        const uint32_t start = tail ? (uint32_t)i * ntail1 : k0[i];
        const bool in = i < nseg && x >= start;
        si = in ? i : si;
        base = in ? start : base;
      }
      key = __builtin_amdgcn_readfirstlane((tail ? kMaxFusedSegs : 0) + si);
      col = (uint32_t)__builtin_amdgcn_readfirstlane((int)((x - base) * (BK * 2)));
    };
    auto col_of = [&](uint32_t c) {
      const uint32_t col = c < nk ? (rotated(c, rot, nk) - (nseg > 1 ? k0_of(k0, key_of(c)) : 0u)) * (BK * 2)
                                  : ((c - nk) % ntail1) * (BK * 2);
      return (uint32_t)__builtin_amdgcn_readfirstlane((int)col);
    };
    for (uint32_t c = 0; c < 2 && c < nsteps; ++c) {
      if (nseg > 1) source(c);
      else if (c == nk) cp = make_acopy(P.At, P.ldat, P.M, m0, cw, lane);
#pragma unroll
      for (int j = 0; j < 8; ++j) a_copy(cp, col_of(c), a_stage(c), cw, j);
    }
    if (nsteps > 1) wait_copies<8>();
    else wait_copies<0>();
    lds_barrier();

    // Step s: slices 0-2 are multiplied while the next slice's fragments are
    // read; the barrier follows; slice 3 is multiplied after it, while the
    // first fragments of step s+1 are read.  Step s+2's eight copies go out
    // two per slice, so six of them are in flight at the barrier that ends
    // step s, by when every copy of step s+1 has landed.  In the last two
    // steps the copies repeat the last step's columns into the stage no one
    // reads (and the last fragment reads fetch a stage no one multiplies), so
    // the loop body has no branch and its order can be fixed: each slice
    // issues the next slice's reads first, then its eight MFMAs with the two
    // copies between them.
    constexpr int kReads = BT ? 8 : 6;  // LDS read instructions per slice
    auto order_slice = [] {
      __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);  // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);       // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);       // copy
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    };
    const uint32_t last_col = col_of(nsteps - 1);
    Frags<BN> cur, nxt;
    load_frags<BN, BT>(cur, a_stage(0), b_stage(0), arow, apos[0], 0);
    for (uint32_t s = 0; s < nsteps; ++s) {
      const uint32_t c = s + 2;
      uint32_t col = last_col;
      if (MULTI) {
        if (c < nsteps) {
          int key;
          key_col(c, key, col);
          source_key(key);
        }
      } else {
        if (c == nk && c < nsteps) cp = make_acopy(P.At, P.ldat, P.M, m0, cw, lane);
        if (c < nsteps) col = col_of(c);
      }
      uint8_t* dst = a_stage(c);
      const uint8_t* As = a_stage(s);
      const uint16_t* Bs = b_stage(s);
#pragma unroll
      for (int ks = 0; ks < 3; ++ks) {
        load_frags<BN, BT>(nxt, As, Bs, arow, apos[ks + 1], ks + 1);
        a_copy(cp, col, dst, cw, 2 * ks);
        a_copy(cp, col, dst, cw, 2 * ks + 1);
        mma_frags<BN>(cur, acc);
        order_slice();
        cur = nxt;
      }
      wait_copies<6>();
      lds_barrier();
      load_frags<BN, BT>(nxt, a_stage(s + 1), b_stage(s + 1), arow, apos[0], 0);
      a_copy(cp, col, dst, cw, 6);
      a_copy(cp, col, dst, cw, 7);
      mma_frags<BN>(cur, acc);
      order_slice();
      cur = nxt;
    }
    // the last copies (into stages no one reads) land before anyone writes
    // the output tile over the A stages: every wave's own, then a barrier
    wait_copies<0>();
    lds_barrier();
    // epilogue: bf16 tile into LDS (over the A stages, no longer read)
    uint16_t* ct = reinterpret_cast<uint16_t*>(lds);
    const int wn = cw & 1;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        // dX: tile column c holds output column 8 (c / 8) + pi(c % 8), the
        // restore's order 0, 2, 4, 6, 1, 3, 5, 7
        const int c = (wn * TN + j) * 32 + (lane & 31);
        const int col = BT ? (c & ~7) | ((c & 3) << 1) | ((c >> 2) & 1) : c;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = (wm * TM + i) * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          ct[row * G::LDC + col] = f32_to_bf16_bits(acc[i][j][v]);
        }
      }
    lds_barrier();
  } else {
    Cursor cur = make_cursor<BN, BT>(P, n0);
    cur.nk = nk;
    cur.rot = rot;
    cur.nseg = (uint32_t)nseg;
#pragma unroll
    for (int i = 0; i <= kMaxFusedSegs; ++i) cur.k0[i] = k0[i];
    cur.lo = 0;
    cur.hi = k0[1];
    auto tail_b = [&](uint32_t s) {
      const uint32_t t = s - nk;
      const int si = __builtin_amdgcn_readfirstlane((int)(t / ntail1));
      const KernargParams K = kernarg_params();
      const uint16_t* bt = si == 0 ? P.Bt : K->seg[si].Bt;
      const int64_t ldbt = si == 0 ? P.ldbt : K->seg[si].ldbt;
      tail_b_store<BN, BT>(bt, ldbt, P.r, P.N, n0, t % ntail1, b_stage(s));
    };
    // three register sets: set i%3 holds step i; in the period of step h the
    // restoring waves issue the loads of step h+3 into the set freed by step
    // h, then restore step h+1 into B stage (h+1)%2, so every load has two
    // steps in flight.
    StepRegs<BN> f0, f1, f2;
    const uint32_t last = nk - 1;
    fetch<BN>(f0, cur, 0, P);
    fetch<BN>(f1, cur, 1 < nk ? 1 : last, P);
    fetch<BN>(f2, cur, 2 < nk ? 2 : last, P);
    restore_step<BN, BT>(f0, P.tab, P.dq, b_stage(0));
    lds_barrier();
    auto period = [&](StepRegs<BN>& into, StepRegs<BN>& from, uint32_t h) {
      fetch<BN>(into, cur, h + 3 < nk ? h + 3 : last, P);
      restore_step<BN, BT>(from, P.tab, P.dq, b_stage(h + 1));
      lds_barrier();
    };
    // periods h = 0 .. nk-2 restore main steps 1 .. nk-1
    for (uint32_t h = 0; h + 1 < nk; h += 6) {
      period(f0, f1, h);
      if (h + 2 < nk) period(f1, f2, h + 1);
      if (h + 3 < nk) period(f2, f0, h + 2);
      if (h + 4 < nk) period(f0, f1, h + 3);
      if (h + 5 < nk) period(f1, f2, h + 4);
      if (h + 6 < nk) period(f2, f0, h + 5);
    }
    // period nk-1 and the tail periods: the rank-r term's B operand
    for (uint32_t h = nk - 1; h < nsteps; ++h) {
      if (h + 1 < nsteps) tail_b(h + 1);
      lds_barrier();
    }
    lds_barrier();  // the multiplying waves' last copies have landed
    lds_barrier();  // the output tile is in LDS
  }

  // coalesced 16-byte stores of the bf16 tile, all eight waves; when
  // accumulating, each 8-element piece is added to C's in fp32 and rounded
  const uint16_t* ct = reinterpret_cast<const uint16_t*>(lds);
  for (int c = threadIdx.x; c < G::BM * (BN / 8); c += 512) {
    const int row = c / (BN / 8), cc = (c % (BN / 8)) * 8;
    const int64_t gr = m0 + row, gc = n0 + cc;
    if (gr >= P.M || gc >= P.N) continue;
    uint4 v = *reinterpret_cast<const uint4*>(ct + row * G::LDC + cc);
    uint4* dst = reinterpret_cast<uint4*>(P.C + gr * P.ldc + gc);
    if (P.accumulate) {
      const uint4 o = *dst;
      const uint32_t ow[4] = {o.x, o.y, o.z, o.w}, nw[4] = {v.x, v.y, v.z, v.w};
      uint32_t sw[4];
#pragma unroll
      for (int h = 0; h < 4; ++h)
        sw[h] = pack_bf16x2(bf16_bits_to_f32(ow[h] & 0xFFFFu) + bf16_bits_to_f32(nw[h] & 0xFFFFu),
                            bf16_bits_to_f32(ow[h] >> 16) + bf16_bits_to_f32(nw[h] >> 16));
      v = make_uint4(sw[0], sw[1], sw[2], sw[3]);
    }
    *dst = v;
  }
}

}  // namespace

__global__ __launch_bounds__(512) void k_qlora_fwd_gemm(FusedParams P) { fused_body<128, false>(P); }
__global__ __launch_bounds__(512) void k_qlora_dx_gemm(FusedParams P) { fused_body<128, true>(P); }
__global__ __launch_bounds__(512) void k_qlora_dx_gemm_multi(FusedParams P) { fused_body<128, true, true>(P); }

hipError_t launch_fused(FusedParams P, bool dx, hipStream_t stream, int kernel_id) {
  if (fused_wide_ok(P, dx)) return launch_fused_wide(P, stream, kernel_id);
  if (!dx && P.nseg > 1) return hipErrorInvalidValue;  // several weights: forward only on 256 x 256 tiles
  constexpr int bn = 128;
  // buffer offsets are 32-bit and the ranges are capped below 2 GiB
  if (P.M * P.lda * 2 > 0x7FFFFFF0LL || (P.r > 0 && P.M * P.ldat * 2 > 0x7FFFFFF0LL) ||
      (dx ? P.K0 : P.N) * P.Kw / 2 > 0x7FFFFFF0LL)
    return hipErrorInvalidValue;
  // QLORA_DX_NARROW=1 keeps dX on the 256 x 128 kernel (to compare the two on one GPU)
  static const bool dx_narrow = [] {
    const char* e = getenv("QLORA_DX_NARROW");
    return e && e[0] == '1';
  }();
  if (dx && !dx_narrow && P.col0 == 0 && fused_dx_wide_ok(P)) {
    // the cheapest of: every tile 256 x 256; whole rounds of those and the
    // rest of dX's columns on this kernel; every tile 256 x 128
    const int64_t mt = (P.M + 255) / 256, nt = (P.N + 255) / 256;
    const int64_t rounds = mt * nt / 256;
    const int64_t ntw = rounds * 256 / mt;
    const int64_t tail_cols = P.N - ntw * 256;
    const int64_t all_wide = wide_cost(mt * nt), all_narrow = narrow_cost(mt * ((P.N + bn - 1) / bn));
    const bool can_split = ntw >= 1 && tail_cols > 0 && mt * nt % 256 != 0;
    const int64_t split = can_split ? 19 * rounds + narrow_cost(mt * ((tail_cols + bn - 1) / bn)) : all_wide + 1;
    if (all_wide <= split && all_wide <= all_narrow) return launch_fused_dx_wide(P, stream, kernel_id);
    if (split < all_narrow) {
      FusedParams W = P;
      W.N = ntw * 256;
      const hipError_t e = launch_fused_dx_wide(W, stream, kernel_id);
      if (e != hipSuccess) return e;
      P.col0 = ntw * 256;
      P.N = tail_cols;
      P.C += P.col0;
      if (P.r > 0) {
        P.Bt += P.col0;
        for (int i = 1; i < P.nseg; ++i) P.seg[i].Bt += P.col0;
      }
    }
  }
  P.mt = (int32_t)((P.M + 255) / 256);
  P.nt = (int32_t)((P.N + bn - 1) / bn);
  P.group_m = 2;
  P.tab = level_table(P.table);
  const int64_t ntiles = (int64_t)P.mt * P.nt;
  const unsigned grid = (unsigned)(((ntiles + 7) / 8) * 8);
  KernelEvents ev(kernel_id);
  if (!dx) hipExtLaunchKernelGGL(k_qlora_fwd_gemm, dim3(grid), dim3(512), 0, stream, ev.start(), ev.stop(), 0, P);
  else if (P.nseg > 1)
    hipExtLaunchKernelGGL(k_qlora_dx_gemm_multi, dim3(grid), dim3(512), 0, stream, ev.start(), ev.stop(), 0, P);
  else hipExtLaunchKernelGGL(k_qlora_dx_gemm, dim3(grid), dim3(512), 0, stream, ev.start(), ev.stop(), 0, P);
  return hipGetLastError();
}

}  // namespace qlora
