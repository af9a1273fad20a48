// The gradient of the layer input on 256 x 256 output tiles:
//   dX = bf16( dY W_hat + [sG_hi | sG_lo] [A ; A] )
//
// "QLoRA技术从入门到精通" §3(2) restores the 4-bit weight to a 16-bit float at
// compute time (table value times the block's stored scale) and discards it;
// the backward of the layer passes the gradient through that restored weight
// ("LoRA 与 QLoRA：把大模型微调拆成可负担的工程", the paragraph on gradients
// through the frozen, dequantized weight).  dX contracts over d_out, the row
// index of the stored weight, so the MFMA's B operand (8 consecutive
// contraction values at one output column per lane) runs across weight rows,
// each of which has its own block scale.  Here every restored block goes into
// an LDS tile in row order, and the fragments are read back transposed
// (ds_read_b64_tr_b16).
//
// Layout of the work (gfx950: one workgroup of four waves per CU, one wave per
// SIMD with 512 registers): workgroup tile 256 tokens x 256 input features;
// wave w multiplies rows 128(w>>1) .. +127 and columns 128(w&1) .. +127
// (4 x 4 tiles of 32 x 32, v_mfma_f32_32x32x16_bf16, 256 fp32 accumulators per
// lane).  Per contraction step of 64 weight rows the same four waves restore
// the whole 64 x 256 B tile of the next step: wave w takes rows 16w .. 16w+15,
// lane l row 16w + l/4 and 64-column block l%4, i.e. one absmax block, so each
// lane builds one table of restored values per step and restores 8 packed
// words (32 bytes, two 16-byte loads).  Each 64 x 256 tile in LDS is moved
// through 192 KB per 2048 MFMA cycles of a SIMD (A copies 32 KB, B stores
// 32 KB, fragment reads 128 KB), against 144 KB per 1024 cycles on 256 x 128
// tiles with separate restoring waves.
//
// B tile (64 rows of 512 B, two stages): 16-byte piece p of row r sits at
// p ^ (p/8 + 4 (r & 1) + 8 ((r >> 1) & 1)).  A restore store (ds_write_b128,
// 8 lanes per cycle on 32 banks: two rows, four blocks, the same piece of
// each) and a transposed fragment read (32 lanes per cycle on 64 banks: four
// rows from a multiple of four, four pieces from a multiple of four) then
// touch each bank once.  Within each group of eight columns the restored
// values stay in nibble order (0, 2, 4, 6, 1, 3, 5, 7; restore8_evenodd), the
// rank-r tail's rows are stored in the same order, and the epilogue puts the
// output columns back.
//
// The activation operand (dY, then the hi/lo pair of s*G for the rank-r tail)
// goes from global memory straight into one of three LDS A stages
// (buffer_load_dwordx4 ... lds), two steps ahead, two copies per slice; A rows
// are 128 B with chunk c of row R at c ^ (R & 7) ^ ((R >> 3) & 1).  One
// barrier per step, in the middle of its last slice: by then every wave has
// stored the next step's B tile and the next step's copies have landed, and
// the last eight MFMAs of the step run while the next step's first fragments
// are read.
//
// Per step s and wave: slice 0 issues the weight loads of step s+2; the
// restore of step s+1 (loaded during step s-1) runs in 39 pieces of a few
// vector instructions, one after each of the 56 MFMAs before the barrier; the
// MFMAs of slices 0-2 are each followed by one fragment read of the next
// slice.  Several weights (the projections that share one input): their
// contraction rows follow each other, each against its own dY, then every
// weight's rank-r tail; dX is one fp32 sum.
#include "fused.hpp"
#include "restore.hpp"
#include "trace.hpp"

namespace qlora {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int A_BYTES = BM * BK * 2;             // one A stage: 256 rows of 128 B
constexpr int B_ROW = BN * 2;                    // 512 B
constexpr int B_BYTES = BK * B_ROW;              // one B stage: 64 rows
constexpr int B_OFF = 3 * A_BYTES;               // the two B stages follow the three A stages
constexpr int MAIN_BYTES = B_OFF + 2 * B_BYTES;  // 160 KB
constexpr int LDC = BN + 8;                      // epilogue bf16 row
constexpr int EPI_BYTES = BM * LDC * 2;
constexpr int LDS_BYTES = MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(4))) FusedParams* KernargParams;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int64_t bytes) {
  const int32_t n = bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0 : (int32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Position of 16-byte piece p (0..31) of B-tile row r.
__device__ __forceinline__ uint32_t bpiece(uint32_t r, uint32_t p) {
  return p ^ ((p >> 3) | ((r & 1u) << 2) | (((r >> 1) & 1u) << 3));
}

// The kernel's one argument, read in place from the kernel-argument segment:
// a field of segment si (wave-uniform, known only at run time) is one scalar
// load at a computed offset.
__device__ __forceinline__ KernargParams kernarg_params() {
  return (KernargParams)__builtin_amdgcn_kernarg_segment_ptr();
}

// Contraction steps: the main steps of weight 0, 1, ... (rotated per tile
// row), then the rank-r tail steps of weight 0, 1, ...  Step c -> its weight
// (si), its step within that weight's rows or tail (local) and its kind.
struct StepMap {
  uint32_t k0[kMaxFusedSegs + 1];  // weight i's first (unrotated) main step; past the last: nk
  uint32_t nk, ntail1, nsteps, rot;
  int nseg;
};

__device__ __forceinline__ void step_of(const StepMap& m, uint32_t c, int& si, uint32_t& local, bool& tail) {
  c = c < m.nsteps ? c : m.nsteps - 1;
  tail = c >= m.nk;
  uint32_t x;
  if (tail) {
    x = c - m.nk;
  } else {
    x = c + m.rot;
    x = x >= m.nk ? x - m.nk : x;
  }
  int s = 0;
  uint32_t base = 0;
#pragma unroll
  for (int i = 1; i < kMaxFusedSegs; ++i) {
    const uint32_t start = tail ? (uint32_t)i * m.ntail1 : m.k0[i];
    const bool in = i < m.nseg && x >= start;
    s = in ? i : s;
    base = in ? start : base;
  }
  si = __builtin_amdgcn_readfirstlane(s);
  local = (uint32_t)__builtin_amdgcn_readfirstlane((int)(x - base));
}

// The rotated position of a main step, advanced one step at a time: x is the
// step's index in the weights' concatenated rows (in 64-row steps), si the
// weight holding it, rows [base, end) of the concatenation that weight's.
struct RunPos {
  uint32_t x, base, end;
  int si;
  __device__ __forceinline__ void set_seg(const StepMap& m, int s) {
    si = s;
    uint32_t b = 0, e = m.k0[1];
#pragma unroll
    for (int i = 1; i < kMaxFusedSegs; ++i) {
      b = s == i ? m.k0[i] : b;
      e = s == i ? m.k0[i + 1] : e;
    }
    base = b;
    end = e;
  }
  __device__ __forceinline__ void init(const StepMap& m, uint32_t c) {
    uint32_t local;
    bool tail;
    int s;
    step_of(m, c, s, local, tail);
    set_seg(m, s);
    x = base + local;
  }
  __device__ __forceinline__ void advance(const StepMap& m) {
    ++x;
    if (x == m.nk) {
      x = 0;
      set_seg(m, 0);
    } else if (x == end) {
      set_seg(m, si + 1);
    }
  }
};

// Weight data of one step for one lane: the 32 packed bytes of its block, the
// aligned dword holding the block's scale code (and the code's bit position),
// the group constant (or the block's fp32 scale without the second level).
struct Fetch {
  u32x4_t w0, w1;
  uint32_t code4, sh;
  float cg;
};

struct WCursor {
  __amdgpu_buffer_rsrc_t rw, rc, rk;
  int seg;           // weight whose resources are loaded (-1: none yet)
  uint32_t woff;     // byte offset of the lane's 32 bytes in the step's first row block
  uint32_t coff;     // 64-weight chunk index of the lane's block in the weight's row rr
  uint32_t kw;       // chunks per step (64 rows x Kw/64)
  uint32_t wstep;    // packed bytes per step (64 rows)
  uint32_t bshift;
};

template <bool DQ>
__device__ __forceinline__ void wcursor_seg(const FusedParams& P, WCursor& c, int si) {
  if (si == c.seg) return;
  c.seg = si;
  const uint8_t* packed;
  const uint8_t* codes;
  const float* consts;
  int64_t rows;
  if (si == 0) {
    packed = P.packed; codes = P.codes; consts = P.consts; rows = P.K0;
  } else {
    const KernargParams K = kernarg_params();
    packed = K->seg[si].packed; codes = K->seg[si].codes; consts = K->seg[si].consts; rows = K->seg[si].N;
  }
  c.rw = rsrc(packed, rows * P.Kw / 2);
  const int64_t nblocks = (rows * P.Kw / 64) >> P.bshift;
  c.rc = rsrc(codes, DQ ? nblocks : 0);
  c.rk = rsrc(consts, DQ ? ((nblocks + 255) / 256) * 4 : nblocks * 4);
}

// The weight loads of main step `local` of weight si: exactly four
// vector-memory loads per call.
template <bool DQ>
__device__ __forceinline__ void fetch_at(Fetch& f, WCursor& c, int si, uint32_t local, const FusedParams& P) {
  wcursor_seg<DQ>(P, c, si);
  const uint32_t sw = local * c.wstep;
  f.w0 = __builtin_amdgcn_raw_buffer_load_b128(c.rw, c.woff, sw, 0);
  f.w1 = __builtin_amdgcn_raw_buffer_load_b128(c.rw, c.woff + 16, sw, 0);
  const uint32_t blk = (c.coff + local * c.kw) >> c.bshift;
  // the codes array holds rows*Kw/blocksize bytes, a multiple of 4, so the aligned
  // dword is in range; without the second level the code load reads zero
  f.code4 = __builtin_amdgcn_raw_buffer_load_b32(c.rc, blk & ~3u, 0, 0);
  f.sh = (blk & 3u) * 8u;
  f.cg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(c.rk, (DQ ? blk >> 8 : blk) * 4, 0, 0));
}

// Keep the scheduler from moving work on fetched registers above their use.
__device__ __forceinline__ void pin(Fetch& f) {
  asm volatile("" : "+v"(f.w0.x), "+v"(f.w0.y), "+v"(f.w0.z), "+v"(f.w0.w));
  asm volatile("" : "+v"(f.w1.x), "+v"(f.w1.y), "+v"(f.w1.z), "+v"(f.w1.w));
  asm volatile("" : "+v"(f.code4), "+v"(f.sh), "+v"(f.cg));
}

// Step kinds of the main loop (see dx_wide_body).
struct Main { static constexpr bool value = true; };
struct Other { static constexpr bool value = false; };
template <int V>
struct Par { static constexpr int value = V; };

__device__ __forceinline__ uint32_t word_of(const Fetch& f, int i) {
  switch (i) {
    case 0: return f.w0.x;
    case 1: return f.w0.y;
    case 2: return f.w0.z;
    case 3: return f.w0.w;
    case 4: return f.w1.x;
    case 5: return f.w1.y;
    case 6: return f.w1.z;
    default: return f.w1.w;
  }
}

// The restore of one step for one lane, cut into 39 pieces of a few vector
// instructions: pieces 0-6 build the block's table (restored scale, the 16
// products and their bf16 pairs, the byte tables), pieces 7 + 4i .. 10 + 4i
// restore word i (restore8_evenodd's steps) and store it.
struct RestoreWork {
  float sc;
  uint32_t w[8];
  RestoreTab t;
  uint32_t sl, s2, HE, LE, HO, LO;
};

template <bool DQ>
__device__ __forceinline__ void restore_piece(int q, const Fetch& f, const Nf4Table& tab, RestoreWork& s,
                                              uint32_t wbase, uint8_t* bst) {
  if (q == 0) {
    s.sc = DQ ? restored_scale((f.code4 >> f.sh) & 0xFFu, f.cg) : f.cg;
  } else if (q <= 4) {
    const int j = 2 * (q - 1);
    s.w[j] = pack_bf16x2(tab.level[2 * j] * s.sc, tab.level[2 * j + 1] * s.sc);
    s.w[j + 1] = pack_bf16x2(tab.level[2 * j + 2] * s.sc, tab.level[2 * j + 3] * s.sc);
  } else if (q <= 6) {
    const int i0 = 2 * (q - 5);
#pragma unroll
    for (int i = i0; i < i0 + 2; ++i) {
      s.t.h[i] = perm(s.w[2 * i + 1], s.w[2 * i], 0x07050301u);
      s.t.l[i] = perm(s.w[2 * i + 1], s.w[2 * i], 0x06040200u);
    }
  } else {
    const int i = (q - 7) >> 2, k = (q - 7) & 3;
    const uint32_t w = word_of(f, i);
    if (k == 0) {
      selectors_even(w, s.sl, s.s2);
      s.HE = perm(perm(s.t.h[3], s.t.h[2], s.sl), perm(s.t.h[1], s.t.h[0], s.sl), s.s2);
    } else if (k == 1) {
      s.LE = perm(perm(s.t.l[3], s.t.l[2], s.sl), perm(s.t.l[1], s.t.l[0], s.sl), s.s2);
      selectors_odd(w, s.sl, s.s2);
    } else if (k == 2) {
      lookup4(s.sl, s.s2, s.t, s.HO, s.LO);
    } else {
      const u32x4_t v = {perm(s.HE, s.LE, 0x05010400u), perm(s.HE, s.LE, 0x07030602u),
                         perm(s.HO, s.LO, 0x05010400u), perm(s.HO, s.LO, 0x07030602u)};
      *reinterpret_cast<u32x4_t*>(bst + (wbase ^ ((uint32_t)i << 4))) = v;
    }
  }
}

// MFMA fragments of one sixteen-wide contraction slice.  The reads take
// restrict-qualified LDS pointers: the stage read is never the one the
// copies in flight are writing (the step's wait and barrier order them), and
// the qualifier keeps the compiler from waiting for every copy before each
// read.
struct Frag {
  bf16x8_t a[4], b[4];
};

// A tile i: row 128wm + 32i + lane%32, chunk 2ks + lane/32 (at byte offset apos)
__device__ __forceinline__ void read_a(Frag& f, const uint8_t* __restrict__ As, uint32_t arow, uint32_t apos, int i) {
  f.a[i] = *reinterpret_cast<const bf16x8_t*>(As + arow + i * 4096 + apos);
}

// B tile j: two transposed reads (contraction rows r .. r+3 and r+4 .. r+7 of
// the lane's column) from the lane's source address at byte offset off
__device__ __forceinline__ void read_b(Frag& f, const uint8_t* __restrict__ Bs, uint32_t off, int j) {
  typedef __attribute__((address_space(3))) uint16_t lds_u16_t;
  const lds_u16_t* p = (const lds_u16_t*)(Bs + off);
  const u16x4_t lo = __builtin_bit_cast(u16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)p));
  const u16x4_t hi = __builtin_bit_cast(u16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(p + 4 * BN)));
  const u16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  f.b[j] = __builtin_bit_cast(bf16x8_t, v);
}

}  // namespace

template <bool DQ, bool SAMELD>
__device__ __forceinline__ void dx_wide_body(const FusedParams& P) {
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
  const int64_t tn = in_group / rows_in_group;
  const int64_t m0 = tm * BM, n0 = tn * BN;

  const int lane = threadIdx.x & 63;
  const int cw = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = cw >> 1, wn = cw & 1;
  const int h = lane >> 5, c32 = lane & 31;

  StepMap sm;
  sm.nseg = P.nseg < 1 ? 1 : P.nseg;
  sm.k0[0] = 0;
  sm.k0[1] = (uint32_t)(P.K0 / BK);
#pragma unroll
  for (int i = 1; i < kMaxFusedSegs; ++i) sm.k0[i + 1] = sm.k0[i] + (i < sm.nseg ? (uint32_t)(P.seg[i].N / BK) : 0u);
  sm.nk = __builtin_amdgcn_readfirstlane(sm.k0[kMaxFusedSegs]);
  sm.ntail1 = P.r > 0 ? (uint32_t)((2 * (int64_t)P.r + BK - 1) / BK) : 0;
  sm.nsteps = __builtin_amdgcn_readfirstlane(sm.nk + sm.ntail1 * (uint32_t)sm.nseg);
  sm.rot = __builtin_amdgcn_readfirstlane((uint32_t)((tm * 5) % sm.nk));
  const uint32_t nk = sm.nk, nsteps = sm.nsteps;

  // the lane's restore unit: row rr of the step, 64-column block b of the tile
  // (blocks beyond the output read block 0 instead: they feed unstored columns)
  const uint32_t rr = (uint32_t)(16 * cw + (lane >> 2)), bb = (uint32_t)(lane & 3);
  const int64_t colb = n0 + 64 * (int64_t)bb < P.N ? (n0 + 64 * (int64_t)bb) / 64 : 0;
  WCursor wc;
  wc.seg = -1;
  wc.woff = (uint32_t)(rr * (P.Kw / 2) + colb * 32);
  wc.coff = (uint32_t)(rr * (P.Kw / 64) + colb);
  wc.kw = (uint32_t)P.Kw;
  wc.wstep = (uint32_t)(32 * P.Kw);
  wc.bshift = (uint32_t)P.bshift;
  const Nf4Table tab = P.tab;
  // byte offset of piece 8b of row rr inside a B stage; piece 8b + i is at wbase ^ 16i
  const uint32_t wbase = rr * B_ROW + bpiece(rr, 8 * bb) * 16;

  // fragment addresses.  A: row 128wm + 32i + c32, chunk 2ks + h.  B (tile j,
  // slice ks): source lane s = lane%16 points at row 16ks + 8h + s/4 (and 4
  // rows further for the second read), column 128wn + 32j + 16((lane>>4)&1) + 4(s%4)
  const uint32_t arow = (uint32_t)((128 * wm + c32) * 128);
  const int x = (c32 & 7) ^ ((c32 >> 3) & 1);
  uint32_t apos[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) apos[ks] = (uint32_t)(((2 * ks + h) ^ x) * 16);
  uint32_t boff[4];
  {
    const uint32_t s16 = (uint32_t)(lane & 15);
    const uint32_t brow = 8u * h + (s16 >> 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t col = 128u * wn + 32u * j + 16u * ((lane >> 4) & 1) + 4u * (s16 & 3);
      boff[j] = brow * B_ROW + bpiece(brow, col >> 3) * 16 + (col & 7) * 2;
    }
  }

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // A copies: copy j of this wave covers rows 64cw + 8j .. +7 of a stage; lane
  // l lands at byte 16l of it (row 64cw + 8j + l/8, position l%8) and so
  // fetches chunk (l%8) ^ (l/8) ^ (j%2) of that row.  Rows beyond the output
  // are clamped to the last row (they only feed output rows never stored).
  uint32_t crow[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t row = m0 + 64 * cw + 8 * j + (lane >> 3);
    crow[j] = (uint32_t)(row < P.M ? row : P.M - 1);
  }
  const uint32_t chunk16[2] = {(uint32_t)(((lane & 7) ^ (lane >> 3)) * 16),
                               (uint32_t)(((lane & 7) ^ (lane >> 3) ^ 1) * 16)};
  // the copy source in use: key si (weight si's dY) or kMaxFusedSegs + si (its hi/lo tail columns)
  int ckey = -1;
  __amdgpu_buffer_rsrc_t rx = rsrc(P.A, 0);
  uint32_t xoff[8];
  auto copy_source = [&](int key) {
    if (key == ckey) return;
    ckey = key;
    const int si = key % kMaxFusedSegs;
    const uint16_t* src;
    int64_t ld;
    if (key < kMaxFusedSegs) {
      if (si == 0) { src = P.A; ld = P.lda; }
      else { const KernargParams K = kernarg_params(); src = K->seg[si].A; ld = K->seg[si].lda; }
    } else {
      if (si == 0) { src = P.At; ld = P.ldat; }
      else { const KernargParams K = kernarg_params(); src = K->seg[si].At; ld = K->seg[si].ldat; }
    }
    rx = rsrc(src, P.M * ld * 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) xoff[j] = crow[j] * (uint32_t)(ld * 2) + chunk16[j & 1];
  };
  // a main step's source inside the loop: with one row stride for every
  // weight's dY (SAMELD) only the scalar resource changes, so the lanes'
  // offsets stay in place from step to step
  auto copy_source_main = [&](int si) {
    if (!SAMELD) {
      copy_source(si);
      return;
    }
    if (si == ckey) return;
    ckey = si;
    const uint16_t* src;
    if (si == 0) src = P.A;
    else { const KernargParams K = kernarg_params(); src = K->seg[si].A; }
    rx = rsrc(src, P.M * P.lda * 2);
  };
  auto stage_a = [&](uint32_t s) { return lds + (s % 3) * A_BYTES; };
  auto stage_b = [&](uint32_t s) { return lds + B_OFF + (s & 1) * B_BYTES; };
  auto copy = [&](uint32_t c, uint32_t col, int j) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(stage_a(c) + (64 * cw + 8 * j) * 128), 16, xoff[j],
                                             col, 0, 0);
  };

  auto rd_a = [&](Frag& f, const uint8_t* As, int ks, int i) { read_a(f, As, arow, apos[ks], i); };
  auto rd_b = [&](Frag& f, const uint8_t* Bs, int ks, int j) { read_b(f, Bs, boff[j] + ks * 16 * B_ROW, j); };
  auto read_frags = [&](Frag& f, uint32_t s, int ks) {
#pragma unroll
    for (int i = 0; i < 4; ++i) rd_a(f, stage_a(s), ks, i);
#pragma unroll
    for (int j = 0; j < 4; ++j) rd_b(f, stage_b(s), ks, j);
  };

  RunPos run;
  // One step s.  MAIN: step s+1 is a weight step, restored from fcur in 39
  // pieces spread over the MFMAs of slices 0-2 and the first half of slice 3;
  // otherwise step s+1 (if any) is a tail step whose B rows (A[kk mod r],
  // kk the tail's contraction index) are loaded at the start and stored in
  // slice 2.  PAR: s mod 2 when known at compile time (0 or 1), else -1.
  // Both kinds issue the weight loads of step s+2 (clamped to the last weight
  // step) into fnext in slice 0 and two copies of step s+2 per slice.  The
  // barrier sits in the middle of slice 3: by then step s+1's copies (issued
  // during step s-1) have landed, since this wave has issued eleven vector-
  // memory operations after them, and every wave has stored step s+1's B
  // tile; the last eight MFMAs of the step run while step s+1's first
  // fragments are read.
  auto step = [&](uint32_t s, Frag& f0, auto main_tag, auto par_tag, auto next_tag, Fetch& fcur, Fetch& fnext) {
    constexpr bool MAIN = decltype(main_tag)::value;
    constexpr int PAR = decltype(par_tag)::value;
    constexpr bool NEXT_MAIN = decltype(next_tag)::value;  // step s+2 is known to be a main step
    uint8_t* const Bc = PAR < 0 ? stage_b(s) : lds + B_OFF + PAR * B_BYTES;
    uint8_t* const Bn = PAR < 0 ? stage_b(s + 1) : lds + B_OFF + (1 - PAR) * B_BYTES;
    const uint8_t* const Ac = stage_a(s);
    const uint8_t* const An = stage_a(s + 1);
    // step s+2: its copies' source and column, and the weight step it loads
    // (a main step: the running position; otherwise the full mapping, with
    // the loads clamped to the last main step)
    int fsi = run.si;
    uint32_t floc = run.x - run.base;
    uint32_t col = floc * (uint32_t)(BK * 2);
    if (NEXT_MAIN) {
      copy_source_main(run.si);
    } else if (s + 2 < nk) {
      copy_source(run.si);
    } else {
      int si2;
      uint32_t loc2;
      bool tail2, t;
      step_of(sm, s + 2, si2, loc2, tail2);
      copy_source((tail2 ? kMaxFusedSegs : 0) + si2);
      col = loc2 * (uint32_t)(BK * 2);
      step_of(sm, nk - 1, fsi, floc, t);
    }
    Frag f1;
    RestoreWork rw;
    u32x4_t tb[8];
    if (!MAIN && s + 1 < nsteps) {
      int si;
      uint32_t local;
      bool tail;
      step_of(sm, s + 1, si, local, tail);
      const uint16_t* bt;
      int64_t ldbt;
      if (si == 0) { bt = P.Bt; ldbt = P.ldbt; }
      else { const KernargParams K = kernarg_params(); bt = K->seg[si].Bt; ldbt = K->seg[si].ldbt; }
      const uint32_t row = (64u * local + rr) % (uint32_t)P.r;
      const uint16_t* src = bt + (int64_t)row * ldbt + colb * 64;
#pragma unroll
      for (int i = 0; i < 8; ++i) tb[i] = *reinterpret_cast<const u32x4_t*>(src + 8 * i);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      Frag& fc = ks % 2 == 0 ? f0 : f1;
      Frag& fn = ks % 2 == 0 ? f1 : f0;
      const int kn = (ks + 1) & 3;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const int i = m >> 2, j = m & 3;
        if (ks == 3 && m == 8) {
          wait_vm<11>();
          lds_barrier();
        }
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fc.a[i], fc.b[j], acc[i][j], 0, 0, 0);
        if (ks < 3) {
          if (m < 4) rd_a(fn, Ac, kn, m);
          else if (m < 8) rd_b(fn, Bc, kn, m - 4);
        } else {
          if (m >= 8 && m < 12) rd_a(fn, An, 0, m - 8);
          else if (m >= 12) rd_b(fn, Bn, 0, m - 12);
        }
        if (m == 4 || m == 12) copy(s + 2, col, 2 * ks + (m == 12));
        if (ks == 0 && m == 1) fetch_at<DQ>(fnext, wc, fsi, floc, P);
        if (MAIN) {
          if (ks == 0 && m == 0) pin(fcur);
          const int g = 16 * ks + m;  // beat; piece q runs in beat 56q/39
#pragma unroll
          for (int q = 0; q < 39; ++q)
            if ((q * 56) / 39 == g) restore_piece<DQ>(q, fcur, tab, rw, wbase, Bn);
        } else if (ks == 2 && m == 8 && s + 1 < nsteps) {
#pragma unroll
          for (int i2 = 0; i2 < 8; ++i2) {
            const u32x4_t v = tb[i2];
            const u32x4_t o = {perm(v.y, v.x, 0x05040100u), perm(v.w, v.z, 0x05040100u),
                               perm(v.y, v.x, 0x07060302u), perm(v.w, v.z, 0x07060302u)};
            *reinterpret_cast<u32x4_t*>(Bn + (wbase ^ ((uint32_t)i2 << 4))) = o;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (s + 2 < nk) run.advance(sm);
  };

  // prologue: weight data of steps 0 and 1, copies of steps 0 and 1, the B
  // tile of step 0, the first fragments
  Fetch F0, F1;
  {
    int si;
    uint32_t local;
    bool tail;
    step_of(sm, 0, si, local, tail);
    fetch_at<DQ>(F0, wc, si, local, P);
    step_of(sm, 1 < nk ? 1 : nk - 1, si, local, tail);
    fetch_at<DQ>(F1, wc, si, local, P);
  }
  for (uint32_t c = 0; c < 2; ++c) {
    int si;
    uint32_t local;
    bool tail;
    step_of(sm, c, si, local, tail);
    copy_source((tail ? kMaxFusedSegs : 0) + si);
#pragma unroll
    for (int j = 0; j < 8; ++j) copy(c, local * (uint32_t)(BK * 2), j);
  }
  {
    RestoreWork rw;
#pragma unroll
    for (int q = 0; q < 39; ++q) restore_piece<DQ>(q, F0, tab, rw, wbase, stage_b(0));
  }
  wait_vm<8>();  // step 0's copies have landed (step 1's may be in flight)
  lds_barrier();
  Frag f0;
  read_frags(f0, 0, 0);

  // the running position of main step 2 (the step whose loads and copies
  // step 0 issues)
  run.init(sm, 2 < nk ? 2 : 0);

  // main steps in pairs (s even, so the B stages' parity is known), then the
  // last main step and the steps whose next step is a tail step (or none)
  // (in the pairs, step s+2 of both steps is a main step; the last main
  // steps may copy a tail step's columns)
  uint32_t s = 0;
  for (; s + 3 < nk; s += 2) {
    step(s, f0, Main{}, Par<0>{}, Main{}, F1, F0);
    step(s + 1, f0, Main{}, Par<1>{}, Main{}, F0, F1);
  }
  if (s + 1 < nk) {
    step(s, f0, Main{}, Par<0>{}, Other{}, F1, F0);
    ++s;
    if (s + 1 < nk) {
      step(s, f0, Main{}, Par<1>{}, Other{}, F0, F1);
      ++s;
    }
  }
  for (; s < nsteps; ++s) step(s, f0, Other{}, Par<-1>{}, Other{}, F1, F0);

  // the last copies (into stages no one reads) land before the output tile
  // goes over the stages: every wave's own, then a barrier
  wait_vm<0>();
  lds_barrier();

  // epilogue: bf16 tile into LDS (tile column c holds output column
  // 8(c/8) + 2(c%4) + (c%8)/4, the restore's order), then coalesced stores;
  // when accumulating, each 8-element piece is added to dX's in fp32 and rounded
  uint16_t* ctile = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 128 * wn + 32 * j + c32;
      const int col = (c & ~7) | ((c & 3) << 1) | ((c >> 2) & 1);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 128 * wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        ctile[row * LDC + col] = f32_to_bf16_bits(acc[i][j][v]);
      }
    }
  lds_barrier();
  for (int c = threadIdx.x; c < BM * (BN / 8); c += 256) {
    const int row = c / (BN / 8), cc = (c % (BN / 8)) * 8;
    const int64_t gr = m0 + row, gc = n0 + cc;
    if (gr >= P.M || gc >= P.N) continue;
    uint4 v = *reinterpret_cast<const uint4*>(ctile + row * LDC + cc);
    uint4* dst = reinterpret_cast<uint4*>(P.C + gr * P.ldc + gc);
    if (P.accumulate) {
      const uint4 o = *dst;
      const uint32_t ow[4] = {o.x, o.y, o.z, o.w}, nw[4] = {v.x, v.y, v.z, v.w};
      uint32_t sw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sw[e] = pack_bf16x2(bf16_bits_to_f32(ow[e] & 0xFFFFu) + bf16_bits_to_f32(nw[e] & 0xFFFFu),
                            bf16_bits_to_f32(ow[e] >> 16) + bf16_bits_to_f32(nw[e] >> 16));
      v = make_uint4(sw[0], sw[1], sw[2], sw[3]);
    }
    *dst = v;
  }
}

// DQ: 8-bit scale codes (else fp32 block scales); _ld: the weights' dY have
// different row strides (several weights of different d_out)
__global__ __launch_bounds__(256, 1) void k_qlora_dx_wide(FusedParams P) { dx_wide_body<true, true>(P); }
__global__ __launch_bounds__(256, 1) void k_qlora_dx_wide_f32s(FusedParams P) { dx_wide_body<false, true>(P); }
__global__ __launch_bounds__(256, 1) void k_qlora_dx_wide_ld(FusedParams P) { dx_wide_body<true, false>(P); }
__global__ __launch_bounds__(256, 1) void k_qlora_dx_wide_f32s_ld(FusedParams P) { dx_wide_body<false, false>(P); }

// 256 x 256 tiles can serve this dX (at least one full round of them; the
// launcher weighs them against the 256 x 128 kernel).  Every weight's rows
// must be whole contraction steps and the output whole 64-column blocks,
// starting at the weight's first column (N may stop short of d_in: the
// 256 x 128 kernel then takes the remaining columns).
bool fused_dx_wide_ok(const FusedParams& P) {
  if (P.K0 % BK != 0 || P.N % 64 != 0 || P.N > P.Kw || P.col0 != 0) return false;
  for (int i = 1; i < P.nseg; ++i)
    if (P.seg[i].N % BK != 0) return false;
  const int64_t mt = (P.M + BM - 1) / BM, nt = (P.N + BN - 1) / BN;
  return mt * nt >= 256;
}

hipError_t launch_fused_dx_wide(FusedParams P, hipStream_t stream, int kernel_id) {
  if (P.nseg < 1) P.nseg = 1;
  P.mt = (int32_t)((P.M + BM - 1) / BM);
  P.nt = (int32_t)((P.N + BN - 1) / BN);
  P.group_m = 2;
  P.tab = level_table(P.table);
  const int64_t ntiles = (int64_t)P.mt * P.nt;
  const unsigned grid = (unsigned)(((ntiles + 7) / 8) * 8);
  bool same_ld = true;
  for (int i = 1; i < P.nseg; ++i) same_ld = same_ld && P.seg[i].lda == P.lda;
  KernelEvents ev(kernel_id);
  auto k = P.dq ? (same_ld ? k_qlora_dx_wide : k_qlora_dx_wide_ld) : (same_ld ? k_qlora_dx_wide_f32s : k_qlora_dx_wide_f32s_ld);
  hipExtLaunchKernelGGL(k, dim3(grid), dim3(256), 0, stream, ev.start(), ev.stop(), 0, P);
  return hipGetLastError();
}

}  // namespace qlora
