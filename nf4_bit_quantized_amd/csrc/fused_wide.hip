// The forward product of the layer on 256 x 256 output tiles, with the NF4
// restore done in registers by the multiplying waves themselves:
//   Y = bf16( X W_hat^T + [sU_hi | sU_lo] [B | B]^T )
//
// "QLoRA技术从入门到精通" §3(2) restores the 4-bit weight to a 16-bit float at
// compute time (table value times the block's stored scale) and discards it;
// here every restored value goes straight from the restoring lane's registers
// into v_mfma_f32_32x32x16_bf16 as its B operand and never reaches LDS or
// memory.
//
// Layout of the work (gfx950: 256 CUs of 4 SIMDs, one workgroup of four waves
// per CU, one wave per SIMD with 512 registers): the workgroup tile is 256
// tokens x 256 output features; wave w owns output features 64w .. 64w+63 for
// all 256 tokens (8 x 2 tiles of 32 x 32, 256 fp32 accumulators per lane).
// No two waves restore the same weight.
//
// The contraction runs in steps of 64 (one absmax block of every weight row).
// The B operand of v_mfma_f32_32x32x16_bf16 gives lane l the 8 contraction
// values 8*(l/32) .. +7 of its slice at column l%32; the order in which a step's
// 64 contraction values enter the four slices is free as long as both operands
// use it, so slice ks of lane half h takes the 8 consecutive values of chunk
// c = 4h + ks.  A lane of half h then needs bytes 16h .. 16h+15 of its weight
// row's 32 packed bytes of the step: one 16-byte load, whose four words are
// its four slices' B fragments once restored (8 indices -> 8 bf16 each).
//
// The activation operand (X, then the hi/lo pair of s*U for the rank-r tail)
// is copied from global memory straight into one of three LDS stages
// (buffer_load_dwordx4 ... lds); each wave copies a quarter of the rows.  A
// rows are 128 B; chunk c of row R sits at position c ^ (R & 7) ^ ((R>>3) & 1),
// so the fragment reads (16 lanes: 16 consecutive rows, one chunk) hit 16
// distinct bank groups.  One barrier per step hands the stages over.
//
// Pipelining per step s (per wave): the A fragments of the next slice are read
// while the current slice's 16 MFMAs run; two of the eight copies for step s+2
// go out per slice; the packed words, scale codes and group constants of step
// s+2 are loaded at the start of the step; the B fragments of step s+1 are
// restored from the words loaded during step s-1, between the MFMAs.
//
// The rank-r term runs as extra contraction steps over the 2r columns of the
// hi/lo split of s*U; its B fragments (B[n][kk mod r]) are loaded from global
// memory directly.  Output: the fp32 tile is rounded to bf16 into LDS and
// written with coalesced 16-byte stores.  The workgroup order is XCD-aware as
// in the 256 x 128 kernel (two tile rows per XCD group, walked column by
// column; rotated contraction start per tile row).
#include "fused.hpp"
#include "restore.hpp"
#include "trace.hpp"

namespace qlora {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int A_BYTES = BM * BK * 2;                 // one A stage: 256 rows of 128 B
constexpr int LDC = BN + 8;                          // epilogue bf16 row
constexpr int EPI_BYTES = BM * LDC * 2;
constexpr int LDS_BYTES = EPI_BYTES > 4 * A_BYTES ? EPI_BYTES : 4 * A_BYTES;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int64_t bytes) {
  const int32_t n = bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0 : (int32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Weight data of one step for one lane: for each of its two 32-column tiles,
// the 16 packed bytes of its half of the row's step segment, the aligned
// dword holding the row block's scale code, and the group constant (or the
// block's fp32 scale without the second level).
struct Fetch {
  u32x4_t w[2];
  uint32_t code4[2];
  float cg[2];
};

struct WCursor {
  __amdgpu_buffer_rsrc_t rw, rc, rk;
  uint32_t woff[2];  // byte offset of the lane's 16 bytes at contraction step 0
  uint32_t coff[2];  // 64-weight chunk index of the lane's row at step 0
  uint32_t nk, rot, bshift;
};

// Steps run in a rotated order per tile row: step s reads column block rot(s).
__device__ __forceinline__ uint32_t rotated(uint32_t step, uint32_t rot, uint32_t nk) {
  const uint32_t kt = step + rot;
  return kt >= nk ? kt - nk : kt;
}

// Exactly six vector-memory loads per call, four with CG (no group constants;
// the waits below count them).
template <bool DQ, bool CG>
__device__ __forceinline__ void fetch(Fetch& f, const WCursor& c, uint32_t step) {
  const uint32_t kt = rotated(step, c.rot, c.nk);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    f.w[j] = __builtin_amdgcn_raw_buffer_load_b128(c.rw, c.woff[j], kt * 32u, 0);
    const uint32_t blk = (c.coff[j] + kt) >> c.bshift;
    // the codes array holds N*K/bs bytes, a multiple of 4, so the aligned dword is in
    // range; without the second level the code load reads zero and cg is the block's scale
    f.code4[j] = __builtin_amdgcn_raw_buffer_load_b32(c.rc, blk & ~3u, 0, 0);
    f.cg[j] = CG ? 0.0f
                 : __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(c.rk, (DQ ? blk >> 8 : blk) * 4, 0, 0));
  }
}

// Bit position of the step's scale code inside the loaded dword.
__device__ __forceinline__ uint32_t code_shift(const WCursor& c, int j, uint32_t step) {
  const uint32_t kt = rotated(step, c.rot, c.nk);
  return (((c.coff[j] + kt) >> c.bshift) & 3u) * 8u;
}

// Keep the scheduler from moving work on fetched registers above their use
// (an early use of a late load would wait for every load issued before it).
__device__ __forceinline__ void pin(Fetch& f) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    asm volatile("" : "+v"(f.w[j].x), "+v"(f.w[j].y), "+v"(f.w[j].z), "+v"(f.w[j].w));
    asm volatile("" : "+v"(f.code4[j]), "+v"(f.cg[j]));
  }
}

struct BFrag {
  bf16x8_t b[2][4];  // [column tile][slice]
};

// The restored scale of the fetched block of column tile j.  CG: every block of
// the lane's row lies in one group of 256, whose step fl32(c_g / 255) the lane
// computed once (step[j]); the result is the same as restored_scale's.
template <bool DQ, bool CG>
__device__ __forceinline__ float fetched_scale(const Fetch& f, int j, uint32_t shift, const float (&step)[2]) {
  if (!DQ) return f.cg[j];
  const uint32_t code = (f.code4[j] >> shift) & 0xFFu;
  return CG ? (float)code * step[j] : restored_scale(code, f.cg[j]);
}

template <bool DQ, bool CG>
__device__ __forceinline__ RestoreTab block_tab(const Fetch& f, int j, uint32_t shift, const Nf4Table& tab,
                                               const float (&step)[2]) {
  return make_tab(tab, fetched_scale<DQ, CG>(f, j, shift, step));
}

__device__ __forceinline__ void restore_word(uint32_t w, const RestoreTab& t, bf16x8_t& out) {
  uint32_t o[4];
  restore8(w, t, o);
  const u32x4_t v = {o[0], o[1], o[2], o[3]};
  out = __builtin_bit_cast(bf16x8_t, v);
}

// The restore of one packed word (restore8) and the table of one block
// (make_tab), cut into pieces of a few vector instructions each, so that a
// wave can place one piece between consecutive MFMAs of its own.  The pieces
// compute exactly what restore8 / make_tab compute.
struct WordWork {
  uint32_t w4, sl, s2, HA, LA, HB, LB;
};

template <int PIECE>
__device__ __forceinline__ void word_piece(uint32_t w, const RestoreTab& t, WordWork& s, bf16x8_t& out) {
  if (PIECE == 0) {  // selectors of elements 0-3
    s.w4 = w >> 4;
    selectors(gather4(w, s.w4, 0), s.sl, s.s2);
  } else if (PIECE == 1) {
    s.HA = perm(perm(t.h[3], t.h[2], s.sl), perm(t.h[1], t.h[0], s.sl), s.s2);
  } else if (PIECE == 2) {
    s.LA = perm(perm(t.l[3], t.l[2], s.sl), perm(t.l[1], t.l[0], s.sl), s.s2);
  } else if (PIECE == 3) {  // selectors of elements 4-7
    selectors(gather4(w, s.w4, 1), s.sl, s.s2);
  } else if (PIECE == 4) {
    lookup4(s.sl, s.s2, t, s.HB, s.LB);
  } else if (PIECE == 5) {  // bf16 pairs (e0,e1) (e2,e3), kept in the same fields
    const uint32_t e01 = perm(s.HA, s.LA, 0x05010400u), e23 = perm(s.HA, s.LA, 0x07030602u);
    s.HA = e01;
    s.LA = e23;
  } else {
    const u32x4_t v = {s.HA, s.LA, perm(s.HB, s.LB, 0x05010400u), perm(s.HB, s.LB, 0x07030602u)};
    out = __builtin_bit_cast(bf16x8_t, v);
  }
}

// The table of a block shared by the two halves of the wave (lanes l and
// l + 32 restore the same weight row, so the same block): each half forms
// the bf16 values of eight of the sixteen levels (half h: levels 8h .. 8h+7,
// lvh = its eight levels), and v_permlane32_swap hands each half the other's.
// Piece 0 forms the restored scale, pieces 1 and 2 four values each, pieces
// 3 and 4 exchange them.  The result equals make_tab's.
struct TabWork {
  float sc;
  uint32_t p[4];
};

template <bool DQ, bool CG, int Q>
__device__ __forceinline__ void tab_piece(const Fetch& f, int j, uint32_t shift, const float (&lvh)[8], TabWork& s,
                                          RestoreTab& t, const float (&step)[2]) {
  if (Q == 0) {
    s.sc = fetched_scale<DQ, CG>(f, j, shift, step);
  } else if (Q == 1 || Q == 2) {
    const int q = Q - 1;
    const uint32_t w0 = pack_bf16x2(lvh[4 * q] * s.sc, lvh[4 * q + 1] * s.sc);
    const uint32_t w1 = pack_bf16x2(lvh[4 * q + 2] * s.sc, lvh[4 * q + 3] * s.sc);
    s.p[2 * q] = perm(w1, w0, 0x07050301u);      // half 0: h[q]; half 1: h[q + 2]
    s.p[2 * q + 1] = perm(w1, w0, 0x06040200u);  // half 0: l[q]; half 1: l[q + 2]
  } else {
    const int q = Q - 3;
    const auto hx = __builtin_amdgcn_permlane32_swap(s.p[2 * q], s.p[2 * q], false, false);
    const auto lx = __builtin_amdgcn_permlane32_swap(s.p[2 * q + 1], s.p[2 * q + 1], false, false);
    t.h[q] = hx[0];
    t.h[q + 2] = hx[1];
    t.l[q] = lx[0];
    t.l[q + 2] = lx[1];
  }
}

// Rank-r tail B fragments of tail step t: B[n][kk mod r], kk = 64t + 8(4h + ks) + e.
// TV: r is a multiple of 8, so each fragment is 8 consecutive elements of B's row.
template <bool TV>
__device__ __forceinline__ void tail_frags(const uint16_t* Bt, int64_t ldbt, int32_t rank, const int64_t (&n)[2], int h,
                                           uint32_t t, BFrag& B) {
  const uint32_t r = (uint32_t)rank;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint16_t* row = Bt + n[j] * ldbt;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint32_t kk = 64u * t + 8u * (4u * h + ks);
      if (TV) {
        B.b[j][ks] = *reinterpret_cast<const bf16x8_t*>(row + kk % r);
      } else {
        uint16_t e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) e[q] = row[(kk + q) % r];
        const u32x4_t v = {e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16),
                           e[4] | ((uint32_t)e[5] << 16), e[6] | ((uint32_t)e[7] << 16)};
        B.b[j][ks] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
  }
}

// Instruction order inside one slice: the next slice's fragment reads and the
// slice's copies (plus, in slice 0, the step's weight loads) first, then the
// 16 MFMAs, each followed by up to V vector instructions of the restore.
template <int KS, int V>
__device__ __forceinline__ void order_slice() {
  __builtin_amdgcn_sched_group_barrier(0x100, KS < 3 ? 8 : 0, 0);  // LDS reads
  __builtin_amdgcn_sched_group_barrier(0x020, KS == 0 ? 8 : 2, 0);  // weight loads (slice 0) and copies
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);  // VALU
  }
}

}  // namespace

template <bool DQ, bool TV, bool CG>
__device__ __forceinline__ void fwd_wide_body(const FusedParams& P) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

  // tile order: chunks of consecutive tiles go to one XCD; inside the order,
  // groups of two tile rows are walked column by column
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
  int64_t tn = in_group / rows_in_group;
  // the weight this tile column belongs to (several weights: their columns follow each other)
  const uint8_t* packed = P.packed;
  const uint8_t* codes = P.codes;
  const float* consts = P.consts;
  int64_t N = P.N;
  const uint16_t* At = P.At;
  int64_t ldat = P.ldat;
  const uint16_t* Bt = P.Bt;
  int64_t ldbt = P.ldbt;
  uint16_t* C = P.C;
  int64_t ldc = P.ldc;
  int64_t first_col = 0;
  for (int i = 1; i < P.nseg; ++i) {
    if (tn >= P.seg_first[i]) {
      const FusedSeg& g = P.seg[i];
      first_col = P.seg_first[i];
      packed = g.packed;
      codes = g.codes;
      consts = g.consts;
      N = g.N;
      At = g.At;
      ldat = g.ldat;
      Bt = g.Bt;
      ldbt = g.ldbt;
      C = g.C;
      ldc = g.ldc;
    }
  }
  tn -= first_col;
  const int64_t m0 = tm * BM, n0 = tn * BN;

  const int lane = threadIdx.x & 63;
  const int cw = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int h = lane >> 5, c32 = lane & 31;
  // step counts and the tile row's rotation are wave-uniform (scalar registers)
  const uint32_t nk = __builtin_amdgcn_readfirstlane((uint32_t)(P.K0 / BK));
  const uint32_t ntail = P.r > 0 ? (uint32_t)((2 * (int64_t)P.r + BK - 1) / BK) : 0;
  const uint32_t nsteps = __builtin_amdgcn_readfirstlane(nk + ntail);
  const uint32_t rot = __builtin_amdgcn_readfirstlane((uint32_t)((tm * 5) % nk));

  // the lane's weight rows (clamped: rows beyond the output feed unstored columns)
  int64_t nrow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = n0 + 64 * cw + 32 * j + c32;
    nrow[j] = n < N ? n : N - 1;
  }
  WCursor wc;
  {
    wc.rw = rsrc(packed, N * P.Kw / 2);
    const int64_t nblocks = (N * P.Kw / 64) >> P.bshift;
    wc.rc = rsrc(codes, DQ ? nblocks : 0);
    wc.rk = rsrc(consts, DQ ? ((nblocks + 255) / 256) * 4 : nblocks * 4);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      wc.woff[j] = (uint32_t)(nrow[j] * (P.Kw / 2) + 16 * h);
      wc.coff[j] = (uint32_t)(nrow[j] * (P.Kw / 64));
    }
    wc.nk = nk;
    wc.rot = rot;
    wc.bshift = (uint32_t)P.bshift;
  }
  // CG: the step fl32(c_g / 255) of each of the lane's two rows' group
  float step[2] = {0.0f, 0.0f};
  if (CG) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      step[j] = scale_step(__builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(wc.rk, ((wc.coff[j] >> wc.bshift) >> 8) * 4, 0, 0)));
  }
  const Nf4Table tab = P.tab;
  float lvh[8];  // the eight levels whose restored values this half of the wave forms
#pragma unroll
  for (int i = 0; i < 8; ++i) lvh[i] = h ? tab.level[8 + i] : tab.level[i];

  // fragment addresses: row 32i + c32, chunk 4h + ks at position (4h + ks) ^ x
  const uint32_t arow = (uint32_t)(c32 * 128);
  const int x = (c32 & 7) ^ ((c32 >> 3) & 1);
  uint32_t apos[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) apos[ks] = (uint32_t)(((4 * h + ks) ^ x) * 16);

  f32x16_t acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // copies: steps < nk read the rotated column block of X, step nk + t the
  // hi/lo columns 64t .. 64t+63; steps past the last repeat the last one.
  // Copy j of this wave covers rows 64cw + 8j .. +7 of the stage: lane l lands
  // at byte 16l of it (row 64cw + 8j + l/8, position l%8) and so fetches
  // chunk (l%8) ^ (l/8) ^ (j%2) of that row.  Rows beyond the output are
  // clamped to the last row (they only feed output rows never stored).
  uint32_t crow[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t row = m0 + 64 * cw + 8 * j + (lane >> 3);
    crow[j] = (uint32_t)(row < P.M ? row : P.M - 1);
  }
  const uint32_t chunk16[2] = {(uint32_t)(((lane & 7) ^ (lane >> 3)) * 16),
                               (uint32_t)(((lane & 7) ^ (lane >> 3) ^ 1) * 16)};
  const __amdgpu_buffer_rsrc_t rx = rsrc(P.A, P.M * P.lda * 2);
  uint32_t xoff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) xoff[j] = crow[j] * (uint32_t)(P.lda * 2) + chunk16[j & 1];
  auto stage = [&](uint32_t s) { return lds + (s & 3) * A_BYTES; };
  auto lds_dst = [&](uint32_t c, int j) { return (lds_void_t*)(stage(c) + (64 * cw + 8 * j) * 128); };
  // copy j of a step c < nk (X)
  auto copy_x = [&](uint32_t c, int j) {
    const uint32_t col = __builtin_amdgcn_readfirstlane(rotated(c, rot, nk) * (BK * 2));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, lds_dst(c, j), 16, xoff[j], col, 0, 0);
  };
  // copy j of any step c (X, or the hi/lo pairs, or a repeat of the last step)
  auto copy = [&](uint32_t c, int j) {
    const uint32_t cc = c < nsteps ? c : nsteps - 1;
    if (cc < nk) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, lds_dst(c, j), 16, xoff[j],
                                               __builtin_amdgcn_readfirstlane(rotated(cc, rot, nk) * (BK * 2)), 0, 0);
    } else {
      const __amdgpu_buffer_rsrc_t rt = rsrc(At, P.M * ldat * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, lds_dst(c, j), 16, crow[j] * (uint32_t)(ldat * 2) + chunk16[j & 1],
                                               __builtin_amdgcn_readfirstlane((cc - nk) * (BK * 2)), 0, 0);
    }
  };
  auto read_a = [&](bf16x8_t (&a)[8], const uint8_t* As, int ks) {
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = *reinterpret_cast<const bf16x8_t*>(As + arow + i * 4096 + apos[ks]);
  };
  auto mma = [&](const bf16x8_t (&a)[8], const BFrag& B, int ks) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], B.b[j][ks], acc[i][j], 0, 0, 0);
  };

  // B fragments of one slice (both column tiles).
  struct BS {
    bf16x8_t b[2];
  };
  auto mma_s = [&](const bf16x8_t (&a)[8], const BS& B) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], B.b[j], acc[i][j], 0, 0, 0);
  };
  auto word = [](const Fetch& f, int j, int ks) {
    return ks == 0 ? f.w[j].x : ks == 1 ? f.w[j].y : ks == 2 ? f.w[j].z : f.w[j].w;
  };
  auto restore_slice = [&](const Fetch& f, const RestoreTab (&t)[2], int ks, BS& out) {
    restore_word(word(f, 0, ks), t[0], out.b[0]);
    restore_word(word(f, 1, ks), t[1], out.b[1]);
  };

  // A weight step s: the B fragments of each slice are restored one slice
  // ahead, between the MFMAs of the slice before.  On entry fa holds step s's
  // weight data (its first slice already restored into b0, with tables t), fb
  // step s+1's (loaded or in flight); step s+2's is loaded into fc in slice 0.
  // Slices 1-3 of step s come from fa; when step s+1 is a weight step, its
  // tables are built from fb in slices 2 and 3 and its first slice restored in
  // slice 3 (into b0 and t for the next step).  Each step issues six weight
  // loads and eight copies, so step s+1's copies (issued during step s-1) have
  // landed once at most 14 vector-memory operations are in flight.
  //
  // Each slice is written as 16 beats, one MFMA each, with the beat's share
  // of the other work after it (one fragment read of the next slice in beats
  // 0-7, a copy in beats 4 and 12, the weight loads in beat 1 of slice 0, one
  // piece of the restore); a scheduling barrier closes every beat, so the
  // vector work of the restore runs beside the MFMAs of the same wave.
  auto weight_step = [&](uint32_t s, bf16x8_t (&a0)[8], const Fetch& fa, Fetch& fb, Fetch& fc, RestoreTab (&t)[2],
                         BS& b0, auto cp) {
    const uint8_t* As = stage(s);
    const uint8_t* An = stage(s + 1);
    bf16x8_t a1[8];
    BS bs[3];
    WordWork w0, w1;
    TabWork tw0, tw1;
    RestoreTab tn[2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8_t(&ac)[8] = ks % 2 == 0 ? a0 : a1;
      bf16x8_t(&an)[8] = ks % 2 == 0 ? a1 : a0;
      const BS& bcur = ks == 0 ? b0 : bs[ks - 1];
      if (ks == 3) {
        // step s+1's copies (issued during step s-2) have landed: after them
        // this wave issued step s-1's six loads (four with CG) and eight
        // copies and six loads (four) and six copies of this step
        wait_vm<CG ? 22 : 26>();
        lds_barrier();
      }
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        acc[m >> 1][m & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ac[m >> 1], bcur.b[m & 1], acc[m >> 1][m & 1], 0, 0, 0);
        // fragments of the next slice; in slice 3, those of step s+1's first slice
        if (m < 8) an[m] = *reinterpret_cast<const bf16x8_t*>((ks < 3 ? As : An) + arow + m * 4096 + apos[(ks + 1) & 3]);
        if (m == 4 || m == 12) cp(s + 3, 2 * ks + (m == 12));
        if (ks == 0 && m == 1) fetch<DQ, CG>(fc, wc, s + 2 < nk ? s + 2 : nk - 1);
        // restore pieces: A = tile 0's word, B = tile 1's
        const uint32_t sh0 = code_shift(wc, 0, s + 1), sh1 = code_shift(wc, 1, s + 1);
        if (ks < 3) {
          // slices 0-2: restore slice ks+1 of step s (pieces of the two tiles
          // alternating in beats 0-13), then pieces of step s+1's tables
          BS& o = bs[ks];
          const uint32_t wa = word(fa, 0, ks + 1), wb = word(fa, 1, ks + 1);
          switch (m) {
            case 0: word_piece<0>(wa, t[0], w0, o.b[0]); break;
            case 1: word_piece<0>(wb, t[1], w1, o.b[1]); break;
            case 2: word_piece<1>(wa, t[0], w0, o.b[0]); break;
            case 3: word_piece<1>(wb, t[1], w1, o.b[1]); break;
            case 4: word_piece<2>(wa, t[0], w0, o.b[0]); break;
            case 5: word_piece<2>(wb, t[1], w1, o.b[1]); break;
            case 6: word_piece<3>(wa, t[0], w0, o.b[0]); break;
            case 7: word_piece<3>(wb, t[1], w1, o.b[1]); break;
            case 8: word_piece<4>(wa, t[0], w0, o.b[0]); break;
            case 9: word_piece<4>(wb, t[1], w1, o.b[1]); break;
            case 10: word_piece<5>(wa, t[0], w0, o.b[0]); break;
            case 11: word_piece<5>(wb, t[1], w1, o.b[1]); break;
            case 12: word_piece<6>(wa, t[0], w0, o.b[0]); break;
            case 13:
              word_piece<6>(wb, t[1], w1, o.b[1]);
              if (ks == 0) pin(fb);
              break;
            case 14:
              if (ks == 0) tab_piece<DQ, CG, 0>(fb, 0, sh0, lvh, tw0, tn[0], step);
              if (ks == 1) tab_piece<DQ, CG, 2>(fb, 0, sh0, lvh, tw0, tn[0], step);
              if (ks == 2) tab_piece<DQ, CG, 4>(fb, 0, sh0, lvh, tw0, tn[0], step);
              break;
            case 15:
              if (ks == 0) tab_piece<DQ, CG, 1>(fb, 0, sh0, lvh, tw0, tn[0], step);
              if (ks == 1) tab_piece<DQ, CG, 3>(fb, 0, sh0, lvh, tw0, tn[0], step);
              if (ks == 2) tab_piece<DQ, CG, 0>(fb, 1, sh1, lvh, tw1, tn[1], step);
              break;
            default: break;
          }
        } else {
          // slice 3: the rest of step s+1's tile 1 table, and step s+1's first slice
          const uint32_t wa = word(fb, 0, 0), wb = word(fb, 1, 0);
          switch (m) {
            case 0: tab_piece<DQ, CG, 1>(fb, 1, sh1, lvh, tw1, tn[1], step); break;
            case 1: word_piece<0>(wa, tn[0], w0, b0.b[0]); break;
            case 2: tab_piece<DQ, CG, 2>(fb, 1, sh1, lvh, tw1, tn[1], step); break;
            case 3: word_piece<1>(wa, tn[0], w0, b0.b[0]); break;
            case 4: tab_piece<DQ, CG, 3>(fb, 1, sh1, lvh, tw1, tn[1], step); break;
            case 5: word_piece<2>(wa, tn[0], w0, b0.b[0]); break;
            case 6: tab_piece<DQ, CG, 4>(fb, 1, sh1, lvh, tw1, tn[1], step); break;
            case 7: word_piece<3>(wa, tn[0], w0, b0.b[0]); break;
            case 8: word_piece<0>(wb, tn[1], w1, b0.b[1]); break;
            case 9: word_piece<4>(wa, tn[0], w0, b0.b[0]); break;
            case 10: word_piece<1>(wb, tn[1], w1, b0.b[1]); break;
            case 11: word_piece<5>(wa, tn[0], w0, b0.b[0]); break;
            case 12: word_piece<2>(wb, tn[1], w1, b0.b[1]); break;
            case 13:
              word_piece<6>(wa, tn[0], w0, b0.b[0]);
              word_piece<3>(wb, tn[1], w1, b0.b[1]);
              break;
            case 14: word_piece<4>(wb, tn[1], w1, b0.b[1]); break;
            case 15:
              word_piece<5>(wb, tn[1], w1, b0.b[1]);
              word_piece<6>(wb, tn[1], w1, b0.b[1]);
              break;
            default: break;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    t[0] = tn[0];
    t[1] = tn[1];
  };

  // The last weight step (its next step is the rank-r tail's, or none) and
  // the tail steps: the same loads, copies and barrier as a weight step, with
  // the B fragments of a tail step (B[n][kk mod r]) loaded during the step
  // before it.  `bnext` receives the next step's fragments when there is one.
  auto plain_step = [&](uint32_t s, bf16x8_t (&a0)[8], auto&& bslice, Fetch& fc, BFrag& bnext) {
    const uint8_t* As = stage(s);
    const uint8_t* An = stage(s + 1);
    bf16x8_t a1[8];
    fetch<DQ, CG>(fc, wc, nk - 1);
    if (s + 1 < nsteps) tail_frags<TV>(Bt, ldbt, P.r, nrow, h, s + 1 - nk, bnext);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks == 3) {
        wait_vm<CG ? 22 : 26>();
        lds_barrier();
      }
      bf16x8_t(&ac)[8] = ks % 2 == 0 ? a0 : a1;
      bf16x8_t(&an)[8] = ks % 2 == 0 ? a1 : a0;
      read_a(an, ks < 3 ? As : An, (ks + 1) & 3);
      copy(s + 3, 2 * ks);
      copy(s + 3, 2 * ks + 1);
      const BS b = bslice(ks);
      mma_s(ac, b);
    }
  };

  // prologue: weight data of steps 0 and 1, copies of steps 0, 1 and 2, the
  // tables and first slice of step 0, and that slice's A fragments
  Fetch fA, fB, fC;
  fetch<DQ, CG>(fA, wc, 0);
  fetch<DQ, CG>(fB, wc, 1 < nk ? 1 : nk - 1);
#pragma unroll
  for (int c = 0; c < 3; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) copy(c, j);
  RestoreTab t[2];
  BS b0;
  t[0] = block_tab<DQ, CG>(fA, 0, code_shift(wc, 0, 0), tab, step);
  t[1] = block_tab<DQ, CG>(fA, 1, code_shift(wc, 1, 0), tab, step);
  restore_slice(fA, t, 0, b0);
  wait_vm<8>();  // steps 0 and 1 have landed (step 2 may be in flight)
  lds_barrier();
  bf16x8_t a0[8];
  read_a(a0, stage(0), 0);

  // weight steps, three per iteration (the weight-data registers rotate)
  // while all copy X for step s+3; then the last ones, whose copies may
  // reach the rank-r tail
  uint32_t s = 0;
  for (; s + 5 < nk; s += 3) {
    weight_step(s, a0, fA, fB, fC, t, b0, copy_x);
    weight_step(s + 1, a0, fB, fC, fA, t, b0, copy_x);
    weight_step(s + 2, a0, fC, fA, fB, t, b0, copy_x);
  }
  for (; s + 1 < nk; ++s) {
    weight_step(s, a0, fA, fB, fC, t, b0, copy);
    const Fetch tmp = fA;
    fA = fB;
    fB = fC;
    fC = tmp;
  }
  {
    // the last weight step: slices 1-3 restored from fA as it goes
    BFrag bn;
    BS bl[4];
    bl[0] = b0;
    restore_slice(fA, t, 1, bl[1]);
    restore_slice(fA, t, 2, bl[2]);
    restore_slice(fA, t, 3, bl[3]);
    plain_step(s, a0, [&](int ks) { return bl[ks]; }, fC, bn);
    ++s;
    // the rank-r tail
    BFrag bc = bn;
    for (; s < nsteps; ++s) {
      plain_step(s, a0, [&](int ks) { BS b; b.b[0] = bc.b[0][ks]; b.b[1] = bc.b[1][ks]; return b; }, fC, bn);
      bc = bn;
    }
  }

  // the last copies (into stages no one reads) land before the output tile
  // goes over the A stages: every wave's own, then a barrier
  wait_vm<0>();
  lds_barrier();

  // epilogue: bf16 tile into LDS, then coalesced 16-byte stores
  uint16_t* ctile = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = 64 * cw + 32 * j + c32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        ctile[row * LDC + col] = f32_to_bf16_bits(acc[i][j][v]);
      }
    }
  lds_barrier();
  for (int c = threadIdx.x; c < BM * (BN / 8); c += 256) {
    const int row = c / (BN / 8), cc = (c % (BN / 8)) * 8;
    const int64_t gr = m0 + row, gc = n0 + cc;
    if (gr >= P.M || gc >= N) continue;
    *reinterpret_cast<uint4*>(C + gr * ldc + gc) = *reinterpret_cast<const uint4*>(ctile + row * LDC + cc);
  }
}

// DQ: 8-bit scale codes (else fp32 block scales); TV: r is a multiple of 8;
// _cg: each weight row's blocks lie in one group of 256 blocks
__global__ __launch_bounds__(256, 1) void k_qlora_fwd_wide(FusedParams P) { fwd_wide_body<true, true, false>(P); }
__global__ __launch_bounds__(256, 1) void k_qlora_fwd_wide_r(FusedParams P) { fwd_wide_body<true, false, false>(P); }
__global__ __launch_bounds__(256, 1) void k_qlora_fwd_wide_cg(FusedParams P) { fwd_wide_body<true, true, true>(P); }
__global__ __launch_bounds__(256, 1) void k_qlora_fwd_wide_r_cg(FusedParams P) { fwd_wide_body<true, false, true>(P); }
__global__ __launch_bounds__(256, 1) void k_qlora_fwd_wide_f32s(FusedParams P) { fwd_wide_body<false, true, false>(P); }
__global__ __launch_bounds__(256, 1) void k_qlora_fwd_wide_f32s_r(FusedParams P) { fwd_wide_body<false, false, false>(P); }

// 256 x 256 tiles where their rounds of the GPU cost no more than those of the
// 256 x 128 kernel's tiles (wide_cost / narrow_cost), or over several weights
// (whose columns must each be whole tiles).
bool fused_wide_ok(const FusedParams& P, bool dx) {
  if (dx || P.accumulate || P.K0 % BK != 0) return false;
  const int64_t mt = (P.M + BM - 1) / BM;
  int64_t nt = (P.N + BN - 1) / BN, nt128 = (P.N + 127) / 128;
  if (P.nseg > 1) {
    if (P.N % BN != 0) return false;
    for (int i = 1; i < P.nseg; ++i) {
      if (P.seg[i].N % BN != 0) return false;
      nt += P.seg[i].N / BN;
      nt128 += P.seg[i].N / 128;
    }
  }
  // several weights: one launch reads X once per tile row (the alternative is
  // a launch per weight), so any full round of tiles takes it
  if (P.nseg > 1) return mt * nt >= 256;
  return mt * nt >= 256 && wide_cost(mt * nt) <= narrow_cost(mt * nt128);
}

hipError_t launch_fused_wide(FusedParams P, hipStream_t stream, int kernel_id) {
  P.mt = (int32_t)((P.M + BM - 1) / BM);
  P.nt = (int32_t)((P.N + BN - 1) / BN);
  if (P.nseg < 1) P.nseg = 1;
  P.seg_first[0] = 0;
  for (int i = 1; i < P.nseg; ++i) {
    P.seg_first[i] = P.nt;
    P.nt += (int32_t)(P.seg[i].N / BN);
  }
  P.seg_first[P.nseg] = P.nt;
  P.group_m = 2;
  P.tab = level_table(P.table);
  const int64_t ntiles = (int64_t)P.mt * P.nt;
  const unsigned grid = (unsigned)(((ntiles + 7) / 8) * 8);
  KernelEvents ev(kernel_id);
  const bool tv = P.r % 8 == 0;
  // blocks per weight row; a row lies in one group of 256 blocks when they divide 256
  const int64_t nbpr = (P.Kw / 64) >> P.bshift;
  const bool cg = nbpr > 0 && 256 % nbpr == 0;
  if (P.dq) {
    auto k = tv ? (cg ? k_qlora_fwd_wide_cg : k_qlora_fwd_wide) : (cg ? k_qlora_fwd_wide_r_cg : k_qlora_fwd_wide_r);
    hipExtLaunchKernelGGL(k, dim3(grid), dim3(256), 0, stream, ev.start(), ev.stop(), 0, P);
  } else {
    if (tv) hipExtLaunchKernelGGL(k_qlora_fwd_wide_f32s, dim3(grid), dim3(256), 0, stream, ev.start(), ev.stop(), 0, P);
    else hipExtLaunchKernelGGL(k_qlora_fwd_wide_f32s_r, dim3(grid), dim3(256), 0, stream, ev.start(), ev.stop(), 0, P);
  }
  return hipGetLastError();
}

}  // namespace qlora
