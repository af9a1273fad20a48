// C ABI of the QLoRA NF4 linear-layer library: validation, workspace
// planning and the sequence of launches on the caller's stream.  The
// declarations, with argument meaning and error behaviour, are in
// include/qlora.h.
#include <cstring>

#include "fused.hpp"
#include "gemm.hpp"
#include "trace.hpp"
#include "../../include/qlora.h"

namespace qlora {
hipError_t launch_nf4_quantize(const float* W, uint8_t* packed, uint8_t* codes, float* consts,
                               int64_t numel, hipStream_t stream);
hipError_t launch_decode(const uint8_t* packed, const uint8_t* codes, const float* consts,
                         const uint16_t* X, int64_t T, int64_t N, int64_t K, int64_t kchunk,
                         int nsplit, float* Ppart, const float* U, int r, float s,
                         const uint16_t* B, uint16_t* Y, hipStream_t stream);
hipError_t launch_reduce_lowrank(const float* P, int nsplit, int64_t split_stride, int64_t T, int r,
                                 float s, float* V, uint16_t* Hs, int64_t ldh, hipStream_t stream);
hipError_t launch_reduce_colpairs(const float* P, int nsplit, int64_t split_stride, int64_t M, int r,
                                  float* out, hipStream_t stream);
hipError_t launch_reduce_rowpairs(const float* P, int nsplit, int64_t split_stride, int r, int64_t K,
                                  float* out, hipStream_t stream);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream);
int gemm_tile_config(int64_t M, int64_t N);
void gemm_tile_shape(int cfg, int* bm, int* bn);
}  // namespace qlora

using namespace qlora;

namespace {

constexpr int64_t kDecodeMaxT = 16;
constexpr int kMaxRank = 128;
constexpr int kTargetWorkgroups = 1024;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int check_desc(const qlora_nf4_desc* d) {
  if (!d) return QLORA_ERR_NULL;
  if (d->blocksize != 64 || d->dq_blocksize != 256) return QLORA_ERR_UNSUPPORTED;
  if (d->d_out <= 0 || d->d_in <= 0 || d->d_out % 64 != 0 || d->d_in % 64 != 0) return QLORA_ERR_SHAPE;
  return QLORA_OK;
}

int check_layer(const qlora_nf4_desc* d, int64_t T, int32_t r) {
  const int st = check_desc(d);
  if (st) return st;
  if (T < 0 || r < 0 || r > kMaxRank) return QLORA_ERR_SHAPE;
  return QLORA_OK;
}

// Split of a partial-sum contraction over grid.z.
struct Split {
  int nsplit;
  int tps;  // 64-wide contraction tiles per split
};

Split plan_split(int64_t M, int64_t N, int64_t kdim) {
  int bm, bn;
  gemm_tile_shape(gemm_tile_config(M, N), &bm, &bn);
  const int64_t tiles = cdiv(M, bm) * cdiv(N, bn);
  const int64_t kt = cdiv(kdim, 64);
  int64_t ns = cdiv(kTargetWorkgroups, tiles);
  const int64_t cap = kt / 2 > 1 ? kt / 2 : 1;
  if (ns > cap) ns = cap;
  if (ns < 1) ns = 1;
  const int64_t tps = cdiv(kt, ns) > 0 ? cdiv(kt, ns) : 1;
  Split s;
  s.tps = (int)tps;
  s.nsplit = (int)(kt > 0 ? cdiv(kt, tps) : 1);
  return s;
}

struct DecodePlan {
  int nsplit;
  int64_t kchunk;
};

DecodePlan plan_decode(int64_t N, int64_t K) {
  const int64_t groups = cdiv(N, 128);
  int64_t ns = cdiv(kTargetWorkgroups, groups);
  if (ns > K / 64) ns = K / 64;
  if (ns < 1) ns = 1;
  DecodePlan p;
  p.kchunk = cdiv(cdiv(K, ns), 64) * 64;
  p.nsplit = (int)cdiv(K, p.kchunk);
  return p;
}

int64_t hilo_ld(int32_t r) { return cdiv(2 * (int64_t)r, 64) * 64; }

// Workspace carving: a bump allocator over the caller's buffer.
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    void* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  }
};

struct FwdWs {
  Split su;
  DecodePlan dp;
  float* u_part = nullptr;
  float* U = nullptr;
  uint16_t* Us = nullptr;
  float* dec = nullptr;
  size_t bytes = 0;
};

FwdWs plan_fwd(const qlora_nf4_desc* d, int64_t T, int32_t r, void* ws) {
  FwdWs w;
  Carve c(ws);
  const int64_t N = d->d_out, K = d->d_in;
  if (r > 0 && T > 0) {
    w.su = plan_split(T, r, K);
    w.u_part = static_cast<float*>(c.take((size_t)w.su.nsplit * T * r * 4));
    w.U = static_cast<float*>(c.take((size_t)T * r * 4));
    w.Us = static_cast<uint16_t*>(c.take((size_t)T * hilo_ld(r) * 2));
  }
  if (T > 0 && T <= kDecodeMaxT) {
    w.dp = plan_decode(N, K);
    w.dec = static_cast<float*>(c.take((size_t)w.dp.nsplit * T * N * 4));
  }
  w.bytes = c.off;
  return w;
}

struct BwdWs {
  Split su, sg, sda, sdb;
  float* u_part = nullptr;
  float* U = nullptr;
  uint16_t* Us = nullptr;
  float* g_part = nullptr;
  uint16_t* Gs = nullptr;
  float* da_part = nullptr;
  float* db_part = nullptr;
  size_t bytes = 0;
};

BwdWs plan_bwd(const qlora_nf4_desc* d, int64_t T, int32_t r, void* ws) {
  BwdWs w;
  Carve c(ws);
  const int64_t N = d->d_out, K = d->d_in;
  if (r > 0 && T > 0) {
    const int64_t ldh = hilo_ld(r);
    w.su = plan_split(T, r, K);
    w.sg = plan_split(T, r, N);
    w.sda = plan_split(2 * (int64_t)r, K, T);
    w.sdb = plan_split(N, 2 * (int64_t)r, T);
    w.u_part = static_cast<float*>(c.take((size_t)w.su.nsplit * T * r * 4));
    w.U = static_cast<float*>(c.take((size_t)T * r * 4));
    w.Us = static_cast<uint16_t*>(c.take((size_t)T * ldh * 2));
    w.g_part = static_cast<float*>(c.take((size_t)w.sg.nsplit * T * r * 4));
    w.Gs = static_cast<uint16_t*>(c.take((size_t)T * ldh * 2));
    w.da_part = static_cast<float*>(c.take((size_t)w.sda.nsplit * 2 * r * K * 4));
    w.db_part = static_cast<float*>(c.take((size_t)w.sdb.nsplit * N * 2 * r * 4));
  }
  w.bytes = c.off;
  return w;
}

Operand op_bf16_k(const uint16_t* p, int64_t ld, int64_t rows, int64_t kdim, int32_t kk_mod = 0) {
  Operand o{};
  o.kind = OP_BF16_K; o.p = p; o.ld = ld; o.rows = rows; o.kdim = kdim; o.kk_mod = kk_mod;
  return o;
}
Operand op_bf16_t(const uint16_t* p, int64_t ld, int64_t rows, int64_t kdim, int32_t kk_mod = 0) {
  Operand o{};
  o.kind = OP_BF16_T; o.p = p; o.ld = ld; o.rows = rows; o.kdim = kdim; o.kk_mod = kk_mod;
  return o;
}
Operand op_nf4(int kind, const uint8_t* packed, const uint8_t* codes, const float* consts, int64_t K,
               int64_t rows, int64_t kdim) {
  Operand o{};
  o.kind = kind; o.p = packed; o.codes = codes; o.consts = consts; o.ld = K; o.rows = rows; o.kdim = kdim;
  return o;
}

GemmParams gemm_one(const Operand& a, const Operand& b, int64_t M, int64_t N) {
  GemmParams p{};
  p.seg[0].a = a; p.seg[0].b = b; p.seg[0].ktiles = cdiv(a.kdim, 64);
  p.nseg = 1; p.M = M; p.N = N; p.nsplit = 1;
  p.tiles_per_split = (int)p.seg[0].ktiles;
  return p;
}

void add_tail(GemmParams& p, const Operand& a, const Operand& b) {
  p.seg[1].a = a; p.seg[1].b = b; p.seg[1].ktiles = cdiv(a.kdim, 64);
  p.nseg = 2;
  p.tiles_per_split = (int)(p.seg[0].ktiles + p.seg[1].ktiles);
}

void out_bf16(GemmParams& p, uint16_t* out, int64_t ldo) {
  p.out_kind = OUT_BF16; p.out = out; p.ldo = ldo;
}

void out_partial(GemmParams& p, float* out, int64_t ldo, const Split& s) {
  p.out_kind = OUT_F32; p.out = out; p.ldo = ldo;
  p.split_stride = p.M * ldo;
  p.nsplit = s.nsplit; p.tiles_per_split = s.tps;
}

#define HIP_TRY(expr)                          \
  do {                                         \
    if ((expr) != hipSuccess) return QLORA_ERR_HIP; \
  } while (0)

// U = X A^T (fp32 into U), and the hi/lo bf16 pair of s*U into Us.
int lora_down(const uint16_t* X, const uint16_t* A, int64_t T, int64_t K, int32_t r, float s,
              const Split& su, float* u_part, float* U, uint16_t* Us, hipStream_t st) {
  GemmParams p = gemm_one(op_bf16_k(X, K, T, K), op_bf16_k(A, K, r, K), T, r);
  out_partial(p, u_part, r, su);
  HIP_TRY(launch_gemm(p, st, KID_LORA_DOWN));
  HIP_TRY(launch_reduce_lowrank(u_part, su.nsplit, (int64_t)T * r, T, r, s, U, Us, hilo_ld(r), st));
  return QLORA_OK;
}

}  // namespace

extern "C" {

const char* qlora_status_string(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_NULL: return "a required pointer is NULL";
    case QLORA_ERR_SHAPE: return "a size is out of range or not a required multiple";
    case QLORA_ERR_UNSUPPORTED: return "unsupported format parameter or pointer alignment";
    case QLORA_ERR_WORKSPACE: return "workspace missing or too small";
    case QLORA_ERR_HIP: return "HIP runtime error while enqueueing work";
    default: return "unknown status";
  }
}

int qlora_nf4_levels(float* levels, float* thresholds) {
  const Nf4Table& t = nf4_table();
  if (levels) std::memcpy(levels, t.level, sizeof(t.level));
  if (thresholds) std::memcpy(thresholds, t.thr, sizeof(t.thr));
  return QLORA_OK;
}

int qlora_nf4_sizes(const qlora_nf4_desc* d, size_t* packed_bytes, size_t* codes_bytes,
                    size_t* consts_bytes) {
  if (!packed_bytes || !codes_bytes || !consts_bytes) return QLORA_ERR_NULL;
  const int st = check_desc(d);
  if (st) return st;
  const int64_t numel = d->d_out * d->d_in;
  const int64_t nb = numel / 64;
  *packed_bytes = (size_t)(numel / 2);
  *codes_bytes = (size_t)nb;
  *consts_bytes = (size_t)cdiv(nb, 256) * 4;
  return QLORA_OK;
}

int qlora_quantize_nf4(const qlora_nf4_desc* d, const float* W, uint8_t* packed, uint8_t* codes,
                       float* consts, void* stream) {
  const int st = check_desc(d);
  if (st) return st;
  if (!W || !packed || !codes || !consts) return QLORA_ERR_NULL;
  if (!aligned16(W) || !aligned16(packed)) return QLORA_ERR_UNSUPPORTED;
  HIP_TRY(launch_nf4_quantize(W, packed, codes, consts, d->d_out * d->d_in, (hipStream_t)stream));
  return QLORA_OK;
}

int qlora_fwd_workspace_bytes(const qlora_nf4_desc* d, int64_t T, int32_t r, size_t* bytes) {
  if (!bytes) return QLORA_ERR_NULL;
  const int st = check_layer(d, T, r);
  if (st) return st;
  *bytes = plan_fwd(d, T, r, nullptr).bytes;
  return QLORA_OK;
}

int qlora_bwd_workspace_bytes(const qlora_nf4_desc* d, int64_t T, int32_t r, size_t* bytes) {
  if (!bytes) return QLORA_ERR_NULL;
  const int st = check_layer(d, T, r);
  if (st) return st;
  *bytes = plan_bwd(d, T, r, nullptr).bytes;
  return QLORA_OK;
}

int qlora_linear_fwd(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes,
                     const float* consts, int64_t T, const uint16_t* X, int32_t r, float alpha,
                     const uint16_t* A, const uint16_t* B, uint16_t* Y, float* U_out,
                     void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_layer(d, T, r);
  if (st) return st;
  if (!packed || !codes || !consts) return QLORA_ERR_NULL;
  if (T > 0 && (!X || !Y)) return QLORA_ERR_NULL;
  if (r > 0 && (!A || !B)) return QLORA_ERR_NULL;
  if (!aligned16(packed) || !aligned16(X) || !aligned16(A)) return QLORA_ERR_UNSUPPORTED;
  const size_t need = plan_fwd(d, T, r, nullptr).bytes;
  if (need > 0 && (!workspace || workspace_bytes < need)) return QLORA_ERR_WORKSPACE;
  if (T == 0) return QLORA_OK;

  hipStream_t s_ = (hipStream_t)stream;
  FwdWs w = plan_fwd(d, T, r, workspace);
  const int64_t N = d->d_out, K = d->d_in;
  const float s = r > 0 ? alpha / (float)r : 0.0f;
  float* U = U_out ? U_out : w.U;

  if (r > 0) {
    const int e = lora_down(X, A, T, K, r, s, w.su, w.u_part, U, w.Us, s_);
    if (e) return e;
  }
  if (T <= kDecodeMaxT) {
    HIP_TRY(launch_decode(packed, codes, consts, X, T, N, K, w.dp.kchunk, w.dp.nsplit, w.dec, U, r, s,
                          B, Y, s_));
    return QLORA_OK;
  }
  FusedParams fp{};
  fp.A = X; fp.lda = K;
  fp.packed = packed; fp.codes = codes; fp.consts = consts; fp.Kw = K;
  fp.M = T; fp.N = N; fp.K0 = K;
  fp.At = w.Us; fp.ldat = hilo_ld(r); fp.Bt = B; fp.ldbt = r; fp.r = r;
  fp.C = Y; fp.ldc = N;
  HIP_TRY(launch_fused(fp, false, s_, KID_FWD_GEMM));
  return QLORA_OK;
}

int qlora_linear_bwd(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes,
                     const float* consts, int64_t T, const uint16_t* X, int32_t r, float alpha,
                     const uint16_t* A, const uint16_t* B, const float* U_in, const uint16_t* dY,
                     uint16_t* dX, float* dA, float* dB, void* workspace, size_t workspace_bytes,
                     void* stream) {
  const int st = check_layer(d, T, r);
  if (st) return st;
  if (!packed || !codes || !consts) return QLORA_ERR_NULL;
  if (T > 0 && (!X || !dY)) return QLORA_ERR_NULL;
  if (r > 0 && (!A || !B || !dA || !dB)) return QLORA_ERR_NULL;
  if (!aligned16(packed) || !aligned16(X) || !aligned16(dY) || !aligned16(A)) return QLORA_ERR_UNSUPPORTED;
  const size_t need = plan_bwd(d, T, r, nullptr).bytes;
  if (need > 0 && (!workspace || workspace_bytes < need)) return QLORA_ERR_WORKSPACE;

  hipStream_t s_ = (hipStream_t)stream;
  const int64_t N = d->d_out, K = d->d_in;
  if (T == 0) {
    if (r > 0) {
      HIP_TRY(launch_fill_zero(dA, (int64_t)r * K, s_));
      HIP_TRY(launch_fill_zero(dB, N * r, s_));
    }
    return QLORA_OK;
  }
  BwdWs w = plan_bwd(d, T, r, workspace);
  const float s = r > 0 ? alpha / (float)r : 0.0f;
  const int64_t ldh = hilo_ld(r);

  if (r > 0) {
    // hi/lo of s*U (recomputing U when it was not saved)
    if (U_in) {
      HIP_TRY(launch_reduce_lowrank(U_in, 1, 0, T, r, s, nullptr, w.Us, ldh, s_));
    } else {
      const int e = lora_down(X, A, T, K, r, s, w.su, w.u_part, w.U, w.Us, s_);
      if (e) return e;
    }
    // G = dY B  ->  hi/lo of s*G
    GemmParams pg = gemm_one(op_bf16_k(dY, N, T, N), op_bf16_t(B, r, r, N), T, r);
    out_partial(pg, w.g_part, r, w.sg);
    HIP_TRY(launch_gemm(pg, s_, KID_LORA_G));
    HIP_TRY(launch_reduce_lowrank(w.g_part, w.sg.nsplit, T * r, T, r, s, nullptr, w.Gs, ldh, s_));
  }
  if (dX) {
    // dX = dY W_hat + (s G) A: the contraction runs over d_out, the rows of W
    FusedParams fp{};
    fp.A = dY; fp.lda = N;
    fp.packed = packed; fp.codes = codes; fp.consts = consts; fp.Kw = K;
    fp.M = T; fp.N = K; fp.K0 = N;
    fp.At = w.Gs; fp.ldat = ldh; fp.Bt = A; fp.ldbt = K; fp.r = r;
    fp.C = dX; fp.ldc = K;
    HIP_TRY(launch_fused(fp, true, s_, KID_DX_GEMM));
  }
  if (r > 0) {
    // dA = (s G)^T X: rows j of the hi/lo pair, contraction over tokens
    GemmParams pa = gemm_one(op_bf16_t(w.Gs, ldh, 2 * (int64_t)r, T), op_bf16_t(X, K, K, T), 2 * (int64_t)r, K);
    out_partial(pa, w.da_part, K, w.sda);
    HIP_TRY(launch_gemm(pa, s_, KID_LORA_DA));
    HIP_TRY(launch_reduce_rowpairs(w.da_part, w.sda.nsplit, 2 * (int64_t)r * K, r, K, dA, s_));
    // dB = dY^T (s U): columns j of the hi/lo pair, contraction over tokens
    GemmParams pb = gemm_one(op_bf16_t(dY, N, N, T), op_bf16_t(w.Us, ldh, 2 * (int64_t)r, T), N, 2 * (int64_t)r);
    out_partial(pb, w.db_part, 2 * (int64_t)r, w.sdb);
    HIP_TRY(launch_gemm(pb, s_, KID_LORA_DB));
    HIP_TRY(launch_reduce_colpairs(w.db_part, w.sdb.nsplit, N * 2 * (int64_t)r, N, r, dB, s_));
  }
  return QLORA_OK;
}

}  // extern "C"
