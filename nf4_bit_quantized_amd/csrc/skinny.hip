// The rank-r adapter products of the layer (skinny: one side is r or 2r wide):
//   forward   U  = X A^T                       [T][r], contraction d_in
//   backward  G  = dY B                        [T][r], contraction d_out
//             dB = dY^T (s U)   (hi+lo pair)   [d_out][r], contraction T
//             dA = (s G)^T X    (hi+lo pair)   [r][d_in],  contraction T
// ("QLoRA技术从入门到精通" §3(2)-(3); "LoRA 与 QLoRA：..." §2: the adapter
// branch is B (A x) scaled by alpha / r; only A and B receive gradients.)
//
// These products read one large operand (X or dY, T x d) once and are bound by
// HBM, not by the matrix cores.  One kernel covers all four:
//   C[m][j] = sum_c Pop[m][c] * Qop[j][c],  m in a 32-row tile, j < J (<= 256)
// Each workgroup owns 32 output rows and all J columns; its four waves split
// the contraction and add their partial tiles through LDS at the end, so no
// partial sums go to memory unless the grid is also split along the
// contraction (then fp32 partials are summed by k_skinny_sum in a fixed order).
// Every 32-wide contraction chunk of each operand is staged by its wave in a
// private LDS slice and read as MFMA fragments, either straight
// (ds_read_b128, contraction contiguous in memory) or transposed
// (ds_read_b64_tr_b16, contraction strided in memory).  v_mfma_f32_16x16x32_bf16,
// fp32 accumulation.
//
// Q operands that hold an fp32 matrix (U saved by the forward) are split into a
// bf16 hi/lo pair while staging: Qop[j][c] = hi(s V[c][j]) for j < r and
// lo(s V[c][j-r]) for r <= j < 2r, so the product carries about 16 bits of
// the fp32 value.
#include <algorithm>

#include "skinny.hpp"
#include "trace.hpp"

namespace qlora {
namespace {

constexpr int CH = 32;     // contraction chunk per MFMA step
constexpr int WAVES = 4;
constexpr int MT = 32;     // output rows per workgroup (two 16-row MFMA tiles)

// contraction chunks a wave loads before using any (register budget:
// (2 + J/16) x 16 B per chunk per lane)
constexpr int chunks_per_wave(int J) { return J <= 64 ? 4 : 2; }

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) uint16_t lds_u16_t;

// Per-wave LDS slice layout (bf16 elements).
template <int J>
struct Slice {
  // contraction-contiguous staging: [rows][CH + 8]; transposed staging: [CH][rows + 16]
  static constexpr int P_ROWS = MT;
  static constexpr int P_ELEMS = (MT * (CH + 8)) > (CH * (MT + 16)) ? MT * (CH + 8) : CH * (MT + 16);
  static constexpr int Q_ELEMS = (J * (CH + 8)) > (CH * (J + 16)) ? J * (CH + 8) : CH * (J + 16);
  static constexpr int ELEMS = P_ELEMS + Q_ELEMS;
};

__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// One contraction chunk of both operands, held in registers between its
// loads and its LDS staging (all of a wave's chunks are loaded up front).
template <int J>
struct ChunkRegs {
  uint4 p[2];        // P: 32 rows x 32 contraction bf16 = 2 KB = 2 x 16 B per lane
  uint4 q[J / 16];   // Q: J rows x 32 bf16, or 32 rows x J/2 fp32 for the hi/lo source
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ uint4 ld8x2(const uint16_t* src, int64_t i0, int64_t limit) {
  uint16_t e[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) e[q] = i0 + q < limit ? src[i0 + q] : (uint16_t)0;
  return make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
}

// Load one 16-byte piece (8 bf16) of a bf16 operand tile.
// CONTIG: piece idx covers (row = idx/4, contraction 8*(idx%4) .. +8) of src[row*ld + c].
// !CONTIG: piece idx covers (contraction c = idx/(ROWS/8), rows 8*(idx%(ROWS/8)) .. +8) of src[c*ld + row].
// Out-of-range rows or contraction positions read as zero.
template <int ROWS, bool CONTIG>
__device__ __forceinline__ uint4 load_piece(const uint16_t* __restrict__ src, int64_t ld, int64_t nrows,
                                            int64_t clen, int64_t r0, int64_t c0, int idx, bool vec) {
  if (CONTIG) {
    const int64_t gr = r0 + (idx >> 2), gc = c0 + (idx & 3) * 8;
    if (gr >= nrows || gc >= clen) return make_uint4(0, 0, 0, 0);
    if (vec && gc + 8 <= clen) return ld16(src + gr * ld + gc);
    return ld8x2(src + gr * ld, gc, clen);
  } else {
    const int64_t gc = c0 + idx / (ROWS / 8), gr = r0 + (idx % (ROWS / 8)) * 8;
    if (gc >= clen || gr >= nrows) return make_uint4(0, 0, 0, 0);
    if (vec && gr + 8 <= nrows) return ld16(src + gc * ld + gr);
    return ld8x2(src + gc * ld, gr, nrows);
  }
}

template <int ROWS, bool CONTIG>
__device__ __forceinline__ void store_piece(uint16_t* __restrict__ dst, int idx, uint4 v) {
  if (CONTIG) *reinterpret_cast<uint4*>(dst + (idx >> 2) * (CH + 8) + (idx & 3) * 8) = v;
  else *reinterpret_cast<uint4*>(dst + (idx / (ROWS / 8)) * (ROWS + 16) + (idx % (ROWS / 8)) * 8) = v;
}

template <int J, bool P_CONTIG, int Q_MODE>
__device__ __forceinline__ void load_chunk(ChunkRegs<J>& R, const SkinnyParams& S, int64_t m0, int64_t c0) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int v = 0; v < 2; ++v)
    R.p[v] = load_piece<MT, P_CONTIG>(S.P, S.ldp, S.mrows, S.clen, m0, c0, lane + 64 * v, S.pvec);
  if (Q_MODE != Q_HILO) {
#pragma unroll
    for (int v = 0; v < J / 16; ++v)
      R.q[v] = load_piece<J, Q_MODE == Q_CONTIG>(S.Q, S.ldq, S.qrows, S.clen, 0, c0, lane + 64 * v, S.qvec);
  } else {
    // fp32 V [c][0..r): 32 rows x r floats; piece idx = 4 floats (row idx/(r/4), cols 4*(idx%(r/4)))
    const int per_row = (S.r + 3) / 4;
#pragma unroll
    for (int v = 0; v < J / 16; ++v) {
      const int idx = lane + 64 * v;
      const int64_t gc = c0 + idx / per_row;
      const int j4 = (idx % per_row) * 4;
      uint4 w = make_uint4(0, 0, 0, 0);
      if (idx < CH * per_row && gc < S.clen) {
        const float* row = S.V + gc * S.ldv;
        float f[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) f[q] = j4 + q < S.r ? row[j4 + q] : 0.0f;
        w = make_uint4(__builtin_bit_cast(uint32_t, f[0]), __builtin_bit_cast(uint32_t, f[1]),
                       __builtin_bit_cast(uint32_t, f[2]), __builtin_bit_cast(uint32_t, f[3]));
      }
      R.q[v] = w;
    }
  }
}

template <int J, bool P_CONTIG, int Q_MODE>
__device__ __forceinline__ void stage_chunk(const ChunkRegs<J>& R, const SkinnyParams& S, uint16_t* __restrict__ Ps,
                                            uint16_t* __restrict__ Qs) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int v = 0; v < 2; ++v) store_piece<MT, P_CONTIG>(Ps, lane + 64 * v, R.p[v]);
  if (Q_MODE != Q_HILO) {
#pragma unroll
    for (int v = 0; v < J / 16; ++v) store_piece<J, Q_MODE == Q_CONTIG>(Qs, lane + 64 * v, R.q[v]);
  } else {
    // hi/lo pair of s*V: Qs[c][j] = hi, Qs[c][r + j] = lo; columns >= 2r stay zero
    const int per_row = (S.r + 3) / 4;
    for (int i = lane; i < CH * (J - 2 * S.r); i += 64) {
      const int c = i / (J - 2 * S.r), j = 2 * S.r + i % (J - 2 * S.r);
      Qs[c * (J + 16) + j] = 0;
    }
#pragma unroll
    for (int v = 0; v < J / 16; ++v) {
      const int idx = lane + 64 * v;
      if (idx >= CH * per_row) continue;
      const int c = idx / per_row, j4 = (idx % per_row) * 4;
      const uint32_t w[4] = {R.q[v].x, R.q[v].y, R.q[v].z, R.q[v].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (j4 + q >= S.r) continue;
        uint16_t hi, lo;
        split_bf16(S.s * __builtin_bit_cast(float, w[q]), hi, lo);
        Qs[c * (J + 16) + j4 + q] = hi;
        Qs[c * (J + 16) + S.r + j4 + q] = lo;
      }
    }
  }
}

// 16x16x32 fragment from a staged tile: rows [row0, row0+16), chunk [0, 32).
template <int ROWS, bool CONTIG>
__device__ __forceinline__ bf16x8_t frag(const uint16_t* __restrict__ t, int row0) {
  const int lane = threadIdx.x & 63;
  if (CONTIG) {
    return *reinterpret_cast<const bf16x8_t*>(t + (row0 + (lane & 15)) * (CH + 8) + 8 * (lane >> 4));
  } else {
    // transposed tile [c][row]: lane group g reads contraction rows 8g..8g+7
    const int s = lane & 15, g = lane >> 4;
    const lds_u16_t* base = (const lds_u16_t*)t;
    const int col = row0 + 4 * (s & 3);
    const int c = 8 * g + (s >> 2);
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(base + c * (ROWS + 16) + col));
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(base + (c + 4) * (ROWS + 16) + col));
    const u16x8_t v = {(uint16_t)lo[0], (uint16_t)lo[1], (uint16_t)lo[2], (uint16_t)lo[3],
                       (uint16_t)hi[0], (uint16_t)hi[1], (uint16_t)hi[2], (uint16_t)hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
  }
}


template <int J, bool P_CONTIG, int Q_MODE>
__global__ __launch_bounds__(256) void k_skinny(SkinnyBatch SB) {
  const SkinnyParams& S = SB.p[blockIdx.z];
  if ((int64_t)blockIdx.x * MT >= S.mrows || (int)blockIdx.y >= S.nsplit) return;
  constexpr int JT = J / 16;
  constexpr int NCH = chunks_per_wave(J);
  using L = Slice<J>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[WAVES * L::ELEMS];
  static_assert(WAVES * L::ELEMS * 2 >= MT * J * 4, "reduction tile fits in the staging space");

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t m0 = (int64_t)blockIdx.x * MT;
  const int z = blockIdx.y;
  uint16_t* Ps = lds + wave * L::ELEMS;
  uint16_t* Qs = Ps + L::P_ELEMS;

  f32x4_t acc[2][JT];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int j = 0; j < JT; ++j) acc[a][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // contraction chunks of this workgroup: split z of S.nsplit; wave w takes
  // chunks cb + w, cb + w + 4, ...
  const int64_t nchunks = (S.clen + CH - 1) / CH;
  const int64_t per = (nchunks + S.nsplit - 1) / S.nsplit;
  const int64_t cb = (int64_t)z * per;
  const int64_t ce = cb + per < nchunks ? cb + per : nchunks;
  // rounds of WAVES * NCH chunks: every chunk of a round is loaded before any is used
  for (int64_t base = cb; base < ce; base += (int64_t)WAVES * NCH) {
    ChunkRegs<J> R[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int64_t ch = base + wave + (int64_t)WAVES * i;
      if (ch < ce) load_chunk<J, P_CONTIG, Q_MODE>(R[i], S, m0, ch * CH);
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int64_t ch = base + wave + (int64_t)WAVES * i;
      if (ch >= ce) break;
      stage_chunk<J, P_CONTIG, Q_MODE>(R[i], S, Ps, Qs);
      wave_lds_sync();
      bf16x8_t pa[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) pa[a] = frag<MT, P_CONTIG>(Ps, 16 * a);
#pragma unroll
      for (int j = 0; j < JT; ++j) {
        const bf16x8_t qb = frag<J, Q_MODE == Q_CONTIG>(Qs, 16 * j);
#pragma unroll
        for (int a = 0; a < 2; ++a) acc[a][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[a], qb, acc[a][j], 0, 0, 0);
      }
      wave_lds_sync();  // fragments read before the slice is overwritten
    }
  }

  // add the four waves' tiles: C[m][j] in fp32, [MT][J]
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);
  for (int w = 0; w < WAVES; ++w) {
    if (wave == w) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int j = 0; j < JT; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * a + 4 * (lane >> 4) + i, col = 16 * j + (lane & 15);
            float* p = red + row * J + col;
            *p = (w == 0 ? 0.0f : *p) + acc[a][j][i];
          }
    }
    __syncthreads();
  }

  // epilogue
  for (int i = threadIdx.x; i < MT * J; i += 256) {
    const int row = i / J, col = i % J;
    const int64_t m = m0 + row;
    if (m >= S.mrows) continue;
    const float v = red[i];
    if (S.out_mode == OUT_PARTIAL) {
      if (col < S.ocols) S.Pout[(int64_t)z * S.mrows * S.ocols + m * S.ocols + col] = v;
    } else if (S.out_mode == OUT_ROWS_HILO) {
      // [T][r] products: optional fp32 copy, hi/lo pair of s*C, zero padding to ldh
      if (col < S.r) {
        if (S.Vout) S.Vout[m * S.r + col] = v;
        uint16_t hi, lo;
        split_bf16(S.s * v, hi, lo);
        S.Hout[m * S.ldh + col] = hi;
        S.Hout[m * S.ldh + S.r + col] = lo;
      }
    } else {
      // pair sums of the hi/lo columns: out[m][col] (dB) or out[col][m] (dA)
      if (col < S.r) {
        const float t = v + red[row * J + col + S.r];
        float* dst = S.out_mode == OUT_PAIRS ? S.Fout + m * S.r + col : S.Fout + (int64_t)col * S.mrows + m;
        *dst = S.accumulate ? *dst + t : t;
      }
    }
  }
  if (S.Ucs && S.nsplit == 1) {
    // hi/lo pair of s * Uc for this workgroup's rows, zero-padded to ldh
    // (with split contractions the sum kernel does this)
    for (int i = threadIdx.x; i < MT * S.ldh; i += 256) {
      const int64_t m = m0 + i / S.ldh;
      const int c = (int)(i % S.ldh);
      if (m >= S.mrows) continue;
      uint16_t h = 0;
      if (c < 2 * S.r) {
        uint16_t hi, lo;
        split_bf16(S.s * S.Uc[m * S.r + (c < S.r ? c : c - S.r)], hi, lo);
        h = c < S.r ? hi : lo;
      }
      S.Ucs[m * S.ldh + c] = h;
    }
  }
  if (S.out_mode == OUT_ROWS_HILO) {
    // zero the padding columns [2r, ldh) of the hi/lo pair
    const int padw = (int)(S.ldh - 2 * S.r);
    for (int i = threadIdx.x; i < MT * padw; i += 256) {
      const int64_t m = m0 + i / padw;
      if (m < S.mrows) S.Hout[m * S.ldh + 2 * S.r + i % padw] = 0;
    }
  }
}

// Fixed-order sum of split partials, then the same outputs as the kernel above.
// TPO threads share one output: thread j adds splits j, j + TPO, ... in order,
// then the TPO sums are added in order (deterministic).  A workgroup covers
// S.sum_per_wg consecutive outputs (at most 256 / TPO); with pairs of columns
// (OUT_PAIRS / OUT_PAIRS_T) that is a whole number of rows, so a row's column
// col + r is in the same workgroup as its column col.
__global__ __launch_bounds__(256) void k_skinny_sum(SkinnyBatch SB, int tpo) {
  const SkinnyParams& S = SB.p[blockIdx.z];
  if (S.nsplit == 1) return;
  __shared__ float part[256];
  __shared__ float tot[256];
  const int per_wg = S.sum_per_wg;
  const int64_t o0 = (int64_t)blockIdx.x * per_wg;
  const int64_t nout = S.mrows * S.ocols;
  if (o0 >= nout) return;
  const int tid = threadIdx.x, o = tid / tpo, j = tid % tpo;
  float v = 0.0f;
  if (o < per_wg && o0 + o < nout)
    for (int z = j; z < S.nsplit; z += tpo) v += S.Pout[(int64_t)z * nout + o0 + o];
  part[tid] = v;
  __syncthreads();
  if (tid < per_wg) {
    float t = 0.0f;
    for (int jj = 0; jj < tpo; ++jj) t += part[tid * tpo + jj];
    tot[tid] = t;
  }
  __syncthreads();
  if (tid >= per_wg || o0 + tid >= nout) return;
  const int64_t idx = o0 + tid;
  const int64_t m = idx / S.ocols;
  const int col = (int)(idx - m * S.ocols);
  if (S.out_mode == OUT_ROWS_HILO) {
    if (col < S.r) {
      const float v2 = tot[tid];
      if (S.Vout) S.Vout[m * S.r + col] = v2;
      uint16_t hi, lo;
      split_bf16(S.s * v2, hi, lo);
      S.Hout[m * S.ldh + col] = hi;
      S.Hout[m * S.ldh + S.r + col] = lo;
    }
    for (int64_t c = 2 * S.r + col; c < S.ldh; c += S.ocols) S.Hout[m * S.ldh + c] = 0;
    if (S.Ucs) {
      if (col < S.r) {
        uint16_t hi, lo;
        split_bf16(S.s * S.Uc[m * S.r + col], hi, lo);
        S.Ucs[m * S.ldh + col] = hi;
        S.Ucs[m * S.ldh + S.r + col] = lo;
      }
      for (int64_t c = 2 * S.r + col; c < S.ldh; c += S.ocols) S.Ucs[m * S.ldh + c] = 0;
    }
  } else if (col < S.r) {
    const float t = tot[tid] + tot[tid + S.r];   // the row's column col + r is in this workgroup
    float* dst = S.out_mode == OUT_PAIRS ? S.Fout + m * S.r + col : S.Fout + (int64_t)col * S.mrows + m;
    *dst = S.accumulate ? *dst + t : t;
  }
}

template <int J, bool P_CONTIG, int Q_MODE>
void launch_j(const SkinnyBatch& S, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((k_skinny<J, P_CONTIG, Q_MODE>), grid, dim3(256), 0, stream, S);
}

template <bool P_CONTIG, int Q_MODE>
void launch_pq(const SkinnyBatch& S, int J, dim3 grid, hipStream_t stream) {
  switch (J) {
    case 32: launch_j<32, P_CONTIG, Q_MODE>(S, grid, stream); break;
    case 64: launch_j<64, P_CONTIG, Q_MODE>(S, grid, stream); break;
    case 128: launch_j<128, P_CONTIG, Q_MODE>(S, grid, stream); break;
    default: launch_j<256, P_CONTIG, Q_MODE>(S, grid, stream); break;
  }
}

}  // namespace

int skinny_width(int cols) { return cols <= 32 ? 32 : cols <= 64 ? 64 : cols <= 128 ? 128 : 256; }

int skinny_splits(int64_t mrows, int64_t clen, int cols) {
  (void)cols;
  const int64_t tiles = (mrows + MT - 1) / MT;
  const int64_t chunks = (clen + CH - 1) / CH;
  // about 512 workgroups in flight, at least one chunk per wave, at most 256
  // partials per output
  int64_t ns = (512 + tiles - 1) / tiles;
  int64_t cap = (chunks + WAVES - 1) / WAVES;
  if (cap > 256) cap = 256;
  if (ns > cap) ns = cap;
  return (int)(ns < 1 ? 1 : ns);
}

namespace {

hipError_t launch_batch(SkinnyBatch B, hipStream_t stream, int kernel_id) {
  const int J = skinny_width(B.p[0].qcols);
  int64_t tiles = 0, ns = 1, outs = 0;
  for (int i = 0; i < B.n; ++i) {
    SkinnyParams& S = B.p[i];
    S.ocols = S.qcols;
    tiles = std::max(tiles, (S.mrows + MT - 1) / MT);
    ns = std::max<int64_t>(ns, S.nsplit);
    if (S.nsplit > 1) outs = std::max(outs, S.mrows * S.ocols);
  }
  // the kernel writes partials whenever it runs split; the sum kernel finishes
  SkinnyBatch K = B;
  for (int i = 0; i < B.n; ++i)
    if (K.p[i].nsplit > 1) K.p[i].out_mode = OUT_PARTIAL;
  const bool p_contig = B.p[0].p_contig;
  const int q_mode = B.p[0].q_mode;
  {
    TraceScope ts(kernel_id, stream);
    const dim3 grid((unsigned)tiles, (unsigned)ns, (unsigned)B.n);
    if (p_contig) {
      if (q_mode == Q_CONTIG) launch_pq<true, Q_CONTIG>(K, J, grid, stream);
      else if (q_mode == Q_STRIDED) launch_pq<true, Q_STRIDED>(K, J, grid, stream);
      else launch_pq<true, Q_HILO>(K, J, grid, stream);
    } else {
      if (q_mode == Q_CONTIG) launch_pq<false, Q_CONTIG>(K, J, grid, stream);
      else if (q_mode == Q_STRIDED) launch_pq<false, Q_STRIDED>(K, J, grid, stream);
      else launch_pq<false, Q_HILO>(K, J, grid, stream);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || outs == 0) return e;
  // threads per output: about 4 splits each, at most 16, and at least one
  // whole row per workgroup when columns are summed in pairs
  int tpo = 1;
  while (tpo < 16 && tpo * 4 < ns) tpo *= 2;
  for (int i = 0; i < B.n; ++i)
    if (B.p[i].out_mode != OUT_ROWS_HILO)
      while (tpo > 1 && 256 / tpo < B.p[i].ocols) tpo /= 2;
  int64_t wgs = 0;
  for (int i = 0; i < B.n; ++i) {
    SkinnyParams& S = B.p[i];
    const int cap = 256 / tpo;
    S.sum_per_wg = S.out_mode == OUT_ROWS_HILO ? cap : (cap / S.ocols) * S.ocols;
    if (S.nsplit > 1) wgs = std::max(wgs, (S.mrows * S.ocols + S.sum_per_wg - 1) / S.sum_per_wg);
  }
  TraceScope ts(KID_REDUCE, stream);
  hipLaunchKernelGGL(k_skinny_sum, dim3((unsigned)wgs, 1, (unsigned)B.n), dim3(256), 0, stream, B, tpo);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny(SkinnyParams S, hipStream_t stream, int kernel_id) {
  SkinnyBatch B{};
  B.p[0] = S;
  B.n = 1;
  return launch_batch(B, stream, kernel_id);
}

hipError_t launch_skinny_pair(SkinnyParams S0, SkinnyParams S1, hipStream_t stream, int kernel_id) {
  if (S0.p_contig != S1.p_contig || S0.q_mode != S1.q_mode || skinny_width(S0.qcols) != skinny_width(S1.qcols))
    return hipErrorInvalidValue;
  SkinnyBatch B{};
  B.p[0] = S0;
  B.p[1] = S1;
  B.n = 2;
  return launch_batch(B, stream, kernel_id);
}

}  // namespace qlora
