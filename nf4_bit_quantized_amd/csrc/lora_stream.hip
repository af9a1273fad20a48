// Streaming kernels for the rank-r adapter products of a layer that sees many
// tokens in one call:
//   rows:  C[m][j] = sum_c P[m][c] Qop[j][c]   U = X A^T, G = dY B   ([T][r])
//   cols:  C[m][j] = sum_t P[t][m] Q[t][j]     dA, dB over the hi/lo pairs
// ("QLoRA技术从入门到精通" §3(2)-(3); "LoRA 与 QLoRA：..." §2: the adapter
// branch is B (A x) scaled by alpha / r; only A and B receive gradients.)
//
// Each product reads one large bf16 matrix (X or dY, T x d) exactly once and is
// bound by HBM.  Unlike the split-contraction kernel in skinny.hip, every
// workgroup here owns whole outputs: its four waves split the contraction and
// add their tiles in LDS in a fixed order, so there are no partial sums in
// memory and no second launch, and results are deterministic.  What keeps HBM
// busy is the number of bytes in flight per CU: each wave keeps several
// contraction chunks loading (registers or LDS copies) while it multiplies an
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

__device__ __forceinline__ f32x4_t mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// rows: C[m][j] = sum_c P[m][c] Qop[j][c], m in RT rows per workgroup, j < r
//
// Contraction chunks of 64 (D is a multiple of 64); wave w takes chunks w,
// w+4, ...  Each chunk of P (RT rows x 128 B) and of Q is copied into LDS.
// Contraction-contiguous tiles (P, and Q = A) keep whole 128-byte rows; the
// sixteen-byte piece p of row R sits at slot p ^ (R & 7) ^ ((R >> 3) & 1), so
// a fragment read (16 lanes: 16 rows, one piece) touches 16 distinct bank
// groups.  Q = B ([D][r], contraction strided) is copied as its contiguous
// [64][r] block and read with transposing LDS reads.
// ---------------------------------------------------------------------------

constexpr int kRowsChunk = 64;

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

template <int JT, bool QS, int RT>
__global__ __launch_bounds__(256) void k_lora_rows(RowsParams p) {
  constexpr int QROWS = 16 * JT;                            // Q tile rows (A) or 64 rows x r (B)
  constexpr int STAGE = RT * 64 + QROWS * 64 + 64;          // bf16 elements (+ slack for transposed reads)
  constexpr int PD0 = (120 * 1024) / (4 * STAGE * 2);
  constexpr int PD = PD0 > 8 ? 8 : PD0;                     // chunks in flight per wave
  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * PD * STAGE];
  __shared__ float red[4][16][16 * JT];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int i = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * RT;
  const int64_t nch = p.D / kRowsChunk;
  const int nmine = nch > wave ? (int)((nch - wave + 3) / 4) : 0;
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
    const int64_t ch = wave + 4 * (int64_t)k;
    const bool in = ch < nch;
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

  // fragment read offsets: row i (P) / Q row j = 16jt + i, pieces 4ks + g
  const int prow_l = i & (RT - 1);
  f32x4_t acc[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) acc[jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

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
        const bf16x8_t a =
            *reinterpret_cast<const bf16x8_t*>(st + prow_l * 64 + ((piece ^ swz(prow_l)) * 8));
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          bf16x8_t b;
          if (QS) {
            b = tr_frag(st + RT * 64, r, 32 * ks + 8 * g, 16 * jt);
          } else {
            const int j = 16 * jt + i < r ? 16 * jt + i : r - 1;
            b = *reinterpret_cast<const bf16x8_t*>(st + RT * 64 + j * 64 + ((piece ^ swz(j)) * 8));
          }
          acc[jt] = mfma(a, b, acc[jt]);
        }
      }
      wait_lds();  // the stage is read before it is refilled
      issue(sp, k + sp + PD);
    }
  }
  wait_vm<0>();

  // fixed-order sum of the four waves' tiles
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][4 * g + v][16 * jt + i] = acc[jt][v];
  __syncthreads();
  const int ldh = (int)p.ldh;
  for (int e = threadIdx.x; e < RT * ldh; e += 256) {
    const int rr = e / ldh, c = e % ldh;
    const int64_t m = m0 + rr;
    if (m >= p.M) continue;
    uint16_t h = 0;
    if (c < 2 * r) {
      const int j = c < r ? c : c - r;
      const float v = ((red[0][rr][j] + red[1][rr][j]) + red[2][rr][j]) + red[3][rr][j];
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
}

// ---------------------------------------------------------------------------
// cols: out[m][j] = sum_t P[t][m] Q[t][j], m in 32 columns per workgroup,
// j < 2r (hi/lo columns of s*G or s*U), then the pair sums.
//
// Contraction chunks of 32 tokens; wave w takes chunks w, w+4, ...  A chunk is
// copied into LDS as two row-major tiles, P [32 t][32 m] and Q [32 t][2r], and
// both MFMA operands are read with transposing LDS reads (their contraction
// runs down the rows).  Workgroups b and b+8 run on the same XCD and take the
// two 64-byte halves of the same 128-byte lines of P.
// ---------------------------------------------------------------------------

template <int J2T>
__global__ __launch_bounds__(256) void k_lora_cols(ColsBatch B) {
  constexpr int J2 = 16 * J2T;
  constexpr int PD = J2T <= 2 ? 6 : (J2T <= 4 ? 4 : 3);  // chunks in flight per wave
  constexpr int NQ = J2T;                                 // Q copies per chunk: 32 x J2 bf16 / 1 KB
  constexpr int STAGE = 32 * 32 + 32 * J2;                // bf16 elements per stage
  constexpr int MAIN = 4 * PD * STAGE * 2;
  constexpr int RED = 4 * 32 * J2 * 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds[MAIN > RED ? MAIN : RED];

  const ColsParams& p = B.p[blockIdx.y];
  const int b = blockIdx.x;
  const int slab = 2 * ((b / 16) * 8 + b % 8) + ((b / 8) & 1);
  const int64_t m0 = (int64_t)slab * 32;
  if (m0 >= p.D) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int g = lane >> 4;
  const int64_t nch = (p.T + 31) / 32;
  const int nmine = nch > wave ? (int)((nch - wave + 3) / 4) : 0;
  const int iters = (nmine + PD - 1) / PD * PD;

  const v4i_t rp = rsrc(p.P, p.T * p.ldp * 2);
  const v4i_t rq = rsrc(p.Q, p.T * p.ldq * 2);
  uint16_t* stage0 = reinterpret_cast<uint16_t*>(lds) + wave * PD * STAGE;
  const uint32_t lstage0 = LDS_ADDR(lds) + (uint32_t)(wave * PD * STAGE * 2);
  // per-lane offsets inside a chunk: P copy q covers tokens 16q + l/4, columns m0 + 8(l%4)
  const uint32_t poff = (uint32_t)((lane >> 2) * p.ldp * 2 + (m0 + 8 * (lane & 3)) * 2);
  auto issue = [&](int sp, int k) {
    const int64_t t0 = (wave + 4 * (int64_t)k) * 32;
    const uint32_t st = lstage0 + (uint32_t)(sp * STAGE * 2);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int64_t t = t0 + 16 * q + (lane >> 2);
      copy16(rp, t < p.T ? (uint32_t)(t0 * p.ldp * 2 + 16 * q * p.ldp * 2) + poff : kOob, st + q * 1024);
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int f = q * 1024 + lane * 16;  // byte of the [32][J2] tile
      const int64_t t = t0 + f / (J2 * 2);
      const uint32_t voff = t < p.T ? (uint32_t)(t * p.ldq * 2 + f % (J2 * 2)) : kOob;
      copy16(rq, voff, st + 2048 + q * 1024);
    }
  };

  f32x4_t acc[2][J2T];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int jt = 0; jt < J2T; ++jt) acc[a][jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int sp = 0; sp < PD; ++sp) issue(sp, sp);
  for (int k = 0; k < iters; k += PD) {
#pragma unroll
    for (int sp = 0; sp < PD; ++sp) {
      wait_vm<(PD - 1) * (2 + NQ)>();  // this chunk's copies have landed
      const uint16_t* st = stage0 + sp * STAGE;
      bf16x8_t pa[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) pa[a] = tr_frag(st, 32, 8 * g, 16 * a);
#pragma unroll
      for (int jt = 0; jt < J2T; ++jt) {
        const bf16x8_t qb = tr_frag(st + 1024, J2, 8 * g, 16 * jt);
#pragma unroll
        for (int a = 0; a < 2; ++a) acc[a][jt] = mfma(pa[a], qb, acc[a][jt]);
      }
      wait_lds();  // the stage is read before it is refilled
      issue(sp, k + sp + PD);
    }
  }
  wait_vm<0>();
  __syncthreads();  // every wave is done with its stages; the space becomes the reduction tile

  float* red = reinterpret_cast<float*>(lds);  // [4][32][J2]
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int jt = 0; jt < J2T; ++jt)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        red[(wave * 32 + 16 * a + 4 * g + v) * J2 + 16 * jt + (lane & 15)] = acc[a][jt][v];
  __syncthreads();
  const int r = p.r;
  for (int e = threadIdx.x; e < 32 * r; e += 256) {
    // dA (transposed output) walks m fastest so its stores are contiguous
    const int mm = p.transposed_out ? e % 32 : e / r;
    const int j = p.transposed_out ? e / 32 : e % r;
    const int64_t m = m0 + mm;
    if (m >= p.D) continue;
    auto col = [&](int jj) {
      return ((red[(0 * 32 + mm) * J2 + jj] + red[(1 * 32 + mm) * J2 + jj]) + red[(2 * 32 + mm) * J2 + jj]) +
             red[(3 * 32 + mm) * J2 + jj];
    };
    const float t = col(j) + col(j + r);
    float* dst = p.transposed_out ? p.Fout + (int64_t)j * p.D + m : p.Fout + m * r + j;
    *dst = p.accumulate ? *dst + t : t;
  }
}

template <bool QS, int RT>
void rows_by_jt(const RowsParams& p, int jt, dim3 grid, hipStream_t st, const KernelEvents& ev) {
  const hipEvent_t e0 = ev.start(), e1 = ev.stop();
  switch (jt) {
    case 1: hipExtLaunchKernelGGL((k_lora_rows<1, QS, RT>), grid, dim3(256), 0, st, e0, e1, 0, p); break;
    case 2: hipExtLaunchKernelGGL((k_lora_rows<2, QS, RT>), grid, dim3(256), 0, st, e0, e1, 0, p); break;
    case 3: hipExtLaunchKernelGGL((k_lora_rows<3, QS, RT>), grid, dim3(256), 0, st, e0, e1, 0, p); break;
    default: hipExtLaunchKernelGGL((k_lora_rows<4, QS, RT>), grid, dim3(256), 0, st, e0, e1, 0, p); break;
  }
}

}  // namespace

int lora_rows_rt(int r) { return r <= 32 ? 8 : 16; }

bool lora_stream_ok(int r) { return r > 0 && r <= 64 && r % 8 == 0; }

bool lora_rows_ok(int64_t M, int r) { return lora_stream_ok(r) && M / lora_rows_rt(r) >= 64; }

hipError_t launch_lora_rows(const RowsParams& p, hipStream_t stream, int kernel_id) {
  if (!lora_rows_ok(p.M, p.r) || p.D % 64 != 0 || p.ldh < 2 * p.r || (p.q_strided && p.ldq != p.r))
    return hipErrorInvalidValue;
  if (p.M * p.ldp * 2 > 0x7FFFFFF0LL || (p.q_strided ? p.D * p.r * 2 : p.r * p.ldq * 2) > 0x7FFFFFF0LL)
    return hipErrorInvalidValue;
  const int rt = lora_rows_rt(p.r);
  const int jt = (p.r + 15) / 16;
  const dim3 grid((unsigned)((p.M + rt - 1) / rt));
  KernelEvents ev(kernel_id);
  if (p.q_strided) {
    if (rt == 8) rows_by_jt<true, 8>(p, jt, grid, stream, ev);
    else rows_by_jt<true, 16>(p, jt, grid, stream, ev);
  } else {
    if (rt == 8) rows_by_jt<false, 8>(p, jt, grid, stream, ev);
    else rows_by_jt<false, 16>(p, jt, grid, stream, ev);
  }
  return hipGetLastError();
}

hipError_t launch_lora_cols(const ColsBatch& B, hipStream_t stream, int kernel_id) {
  int64_t slabs = 0;
  for (int k = 0; k < B.n; ++k) {
    const ColsParams& p = B.p[k];
    if (p.r != B.p[0].r || !lora_stream_ok(p.r) || p.D % 32 != 0 || p.ldq < 2 * p.r) return hipErrorInvalidValue;
    if (p.T * p.ldp * 2 > 0x7FFFFFF0LL || p.T * p.ldq * 2 > 0x7FFFFFF0LL) return hipErrorInvalidValue;
    slabs = std::max<int64_t>(slabs, p.D / 32);
  }
  const dim3 grid((unsigned)((slabs + 15) / 16 * 16), (unsigned)B.n);
  KernelEvents ev(kernel_id);
  const hipEvent_t e0 = ev.start(), e1 = ev.stop();
  switch (B.p[0].r / 8) {
    case 1: hipExtLaunchKernelGGL(k_lora_cols<1>, grid, dim3(256), 0, stream, e0, e1, 0, B); break;
    case 2: hipExtLaunchKernelGGL(k_lora_cols<2>, grid, dim3(256), 0, stream, e0, e1, 0, B); break;
    case 3: hipExtLaunchKernelGGL(k_lora_cols<3>, grid, dim3(256), 0, stream, e0, e1, 0, B); break;
    case 4: hipExtLaunchKernelGGL(k_lora_cols<4>, grid, dim3(256), 0, stream, e0, e1, 0, B); break;
    case 5: hipExtLaunchKernelGGL(k_lora_cols<5>, grid, dim3(256), 0, stream, e0, e1, 0, B); break;
    case 6: hipExtLaunchKernelGGL(k_lora_cols<6>, grid, dim3(256), 0, stream, e0, e1, 0, B); break;
    case 7: hipExtLaunchKernelGGL(k_lora_cols<7>, grid, dim3(256), 0, stream, e0, e1, 0, B); break;
    default: hipExtLaunchKernelGGL(k_lora_cols<8>, grid, dim3(256), 0, stream, e0, e1, 0, B); break;
  }
  return hipGetLastError();
}

}  // namespace qlora
