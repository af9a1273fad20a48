// C ABI of the QLoRA NF4 linear-layer library: validation, workspace
// planning and the sequence of launches on the caller's stream.  The
// declarations, with argument meaning and error behaviour, are in
// include/qlora.h.
#include <algorithm>
#include <cstring>
#include <mutex>

#include "fused.hpp"
#include "lora_stream.hpp"
#include <cmath>

#include "adamw.hpp"
#include "decode.hpp"
#include "dropout.hpp"
#include "skinny.hpp"
#include "trace.hpp"
#include "../../include/qlora.h"

namespace qlora {
hipError_t launch_nf4_quantize(const void* W, int wformat, uint8_t* packed, uint8_t* codes, float* consts,
                               int64_t numel, int blocksize, int dq, int table, hipStream_t stream);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream);
hipError_t launch_export(const uint8_t* packed, const uint8_t* codes, const float* consts, int64_t N, int64_t K,
                         int r, float s, const uint16_t* A, const uint16_t* B, uint16_t* W, int table,
                         int bshift, int dq, hipStream_t stream);
}  // namespace qlora

using namespace qlora;

namespace {

constexpr int64_t kDecodeMaxT = 16;
constexpr int kMaxRank = 128;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// log2(blocksize / 64): 64-weight chunk index -> block index
int block_shift(const qlora_nf4_desc* d) { return d->blocksize == 256 ? 2 : (d->blocksize == 128 ? 1 : 0); }

// The few-token kernel takes this weight (8-bit codes are staged from a
// 16-byte aligned run; fp32 block scales are read per chunk).
bool decode_ok(const qlora_nf4_desc* d, const uint8_t* codes, const float* consts) {
  const bool f32s = d->dq_blocksize == 0;
  return decode_supported(d->d_out, d->d_in, block_shift(d), f32s) && (f32s ? aligned16(consts) : aligned16(codes));
}

int check_desc(const qlora_nf4_desc* d) {
  if (!d) return QLORA_ERR_NULL;
  if ((d->blocksize != 64 && d->blocksize != 128 && d->blocksize != 256) ||
      (d->dq_blocksize != 256 && d->dq_blocksize != 0))
    return QLORA_ERR_UNSUPPORTED;
  if (d->table != QLORA_TABLE_NF4 && d->table != QLORA_TABLE_UNIFORM) return QLORA_ERR_UNSUPPORTED;
  if (d->d_out <= 0 || d->d_in <= 0 || d->d_out % 64 != 0 || d->d_in % 64 != 0) return QLORA_ERR_SHAPE;
  return QLORA_OK;
}

int64_t hilo_ld(int32_t r) { return cdiv(2 * (int64_t)r, 64) * 64; }

// The kernels address every dense operand with 32-bit byte offsets (buffer
// resources capped below 2 GiB): the packed weight, X, Y, dY, dX and the
// workspace's [T][2r] pairs must each stay below kMaxOperandBytes.
constexpr int64_t kMaxOperandBytes = 0x7FFFFFF0LL;
constexpr int64_t kMaxDim = (int64_t)1 << 31;

int check_layer(const qlora_nf4_desc* d, int64_t T, int32_t r) {
  const int st = check_desc(d);
  if (st) return st;
  if (T < 0 || r < 0 || r > kMaxRank) return QLORA_ERR_SHAPE;
  const int64_t N = d->d_out, K = d->d_in;
  if (N >= kMaxDim || K >= kMaxDim || T >= kMaxDim) return QLORA_ERR_SHAPE;
  if (N * K / 2 > kMaxOperandBytes || T * K * 2 > kMaxOperandBytes || T * N * 2 > kMaxOperandBytes ||
      T * hilo_ld(r) * 2 > kMaxOperandBytes)
    return QLORA_ERR_SHAPE;
  return QLORA_OK;
}

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

// Scratch for the split-contraction partials of one rank-r product.
size_t skinny_part_bytes(int64_t mrows, int64_t clen, int64_t cols) {
  const int ns = skinny_splits(mrows, clen, (int)cols);
  return ns > 1 ? (size_t)ns * mrows * cols * 4 : 0;
}

struct FwdWs {
  float* part = nullptr;
  float* U = nullptr;
  uint16_t* Us = nullptr;
  float* dpart = nullptr;  // the few-token kernel's contraction-split sums
  size_t dpart_bytes = 0;
  size_t bytes = 0;
};

FwdWs plan_fwd(const qlora_nf4_desc* d, int64_t T, int32_t r, void* ws) {
  FwdWs w;
  Carve c(ws);
  const int64_t N = d->d_out, K = d->d_in;
  if (r > 0 && T > 0) {
    w.part = static_cast<float*>(
        c.take(lora_rows_ok(T, r) ? lora_rows_part_bytes(T, K, r) : skinny_part_bytes(T, K, r)));
    w.U = static_cast<float*>(c.take((size_t)T * r * 4));
    w.Us = static_cast<uint16_t*>(c.take((size_t)T * hilo_ld(r) * 2));
  }
  if (T > 0 && T <= kDecodeMaxT) {
    w.dpart_bytes = decode_part_bytes(T, N, K, block_shift(d), d->dq_blocksize == 0);
    w.dpart = static_cast<float*>(c.take(w.dpart_bytes));
  }
  w.bytes = c.off;
  return w;
}

struct BwdWs {
  float* part = nullptr;   // shared by the rank-r products that run one after another
  float* part2 = nullptr;  // dB's partials (it runs in the same launch as dA)
  size_t part_bytes = 0;
  float* U = nullptr;
  uint16_t* Us = nullptr;
  uint16_t* Gs = nullptr;
  size_t bytes = 0;
};

BwdWs plan_bwd(const qlora_nf4_desc* d, int64_t T, int32_t r, void* ws) {
  BwdWs w;
  Carve c(ws);
  const int64_t N = d->d_out, K = d->d_in;
  if (r > 0 && T > 0) {
    const int64_t ldh = hilo_ld(r);
    // split-contraction partials, only for the products the streaming kernels do not take
    size_t part = 0, part2 = 0;
    // (U's and G's: the streaming kernel's contraction-range partials, or the skinny kernel's)
    if (!lora_rows_ok(T, r)) part = std::max(skinny_part_bytes(T, K, r), skinny_part_bytes(T, N, r));
    else part = std::max(lora_rows_part_bytes(T, K, r), lora_rows_part_bytes(T, N, r));
    if (!lora_stream_ok(r)) {
      part = std::max(part, skinny_part_bytes(K, T, 2 * (int64_t)r));
      part2 = skinny_part_bytes(N, T, 2 * (int64_t)r);
    } else {
      // the streaming dA/dB kernel's token-range partials (it runs after G is done with part)
      const int64_t Ds[2] = {K, N};
      part = std::max(part, lora_cols_part_bytes(T, Ds, 2, r));
    }
    w.part_bytes = part;
    w.part = static_cast<float*>(c.take(part));
    w.part2 = static_cast<float*>(c.take(part2));
    w.U = static_cast<float*>(c.take((size_t)T * r * 4));
    w.Us = static_cast<uint16_t*>(c.take((size_t)T * ldh * 2));
    w.Gs = static_cast<uint16_t*>(c.take((size_t)T * ldh * 2));
  }
  w.bytes = c.off;
  return w;
}

bool vec_ok(const void* p, int64_t ld) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0 && (ld & 7) == 0; }

SkinnyParams skinny(const uint16_t* P, int64_t ldp, bool p_contig, int64_t mrows, int64_t clen, int r, float s,
                    int qcols, int out_mode, float* part) {
  SkinnyParams S{};
  S.P = P; S.ldp = ldp; S.p_contig = p_contig; S.pvec = vec_ok(P, ldp);
  S.mrows = mrows; S.clen = clen; S.r = r; S.s = s; S.qcols = qcols; S.out_mode = out_mode;
  S.nsplit = skinny_splits(mrows, clen, qcols);
  S.Pout = part;
  return S;
}

void skinny_q(SkinnyParams& S, const uint16_t* Q, int64_t ldq, int64_t qrows, int q_mode) {
  S.Q = Q; S.ldq = ldq; S.qrows = qrows; S.q_mode = q_mode; S.qvec = vec_ok(Q, ldq);
}

#define HIP_TRY(expr)                          \
  do {                                         \
    if ((expr) != hipSuccess) return QLORA_ERR_HIP; \
  } while (0)

// U = X A^T (fp32 into U), and the hi/lo bf16 pair of s*U into Us.
int lora_down(const uint16_t* X, const uint16_t* A, int64_t T, int64_t K, int32_t r, float s, float* part,
              float* U, uint16_t* Us, hipStream_t st) {
  if (lora_down_small_ok(T, K, r)) {  // few tokens: one launch, no partial sums
    const SmallDownParams P{X, A, T, K, r, s, U, Us, hilo_ld(r)};
    HIP_TRY(launch_lora_down_small(P, st, KID_LORA_DOWN));
    return QLORA_OK;
  }
  if (lora_rows_ok(T, r)) {
    RowsParams R{};
    R.P = X; R.ldp = K; R.M = T; R.D = K;
    R.Q = A; R.ldq = K; R.q_strided = 0; R.r = r; R.s = s;
    R.Vout = U; R.Hout = Us; R.ldh = hilo_ld(r);
    HIP_TRY(launch_lora_rows(R, part, lora_rows_part_bytes(T, K, r), st, KID_LORA_DOWN));
    return QLORA_OK;
  }
  SkinnyParams S = skinny(X, K, true, T, K, r, s, r, OUT_ROWS_HILO, part);
  skinny_q(S, A, K, r, Q_CONTIG);
  S.Vout = U; S.Hout = Us; S.ldh = hilo_ld(r);
  HIP_TRY(launch_skinny(S, st, KID_LORA_DOWN));
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
    case QLORA_ERR_SCRATCH_LIMIT: return "the call needs more scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

int qlora_nf4_levels(float* levels, float* thresholds) { return qlora_table_levels(QLORA_TABLE_NF4, levels, thresholds); }

int qlora_table_levels(int32_t table, float* levels, float* thresholds) {
  if (table != QLORA_TABLE_NF4 && table != QLORA_TABLE_UNIFORM) return QLORA_ERR_UNSUPPORTED;
  const Nf4Table& t = level_table(table);
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
  const int64_t nb = numel / d->blocksize;
  *packed_bytes = (size_t)(numel / 2);
  const bool dq = d->dq_blocksize != 0;
  *codes_bytes = dq ? (size_t)nb : 0;
  *consts_bytes = dq ? (size_t)cdiv(nb, 256) * 4 : (size_t)nb * 4;
  return QLORA_OK;
}

int qlora_quantize_nf4(const qlora_nf4_desc* d, const float* W, uint8_t* packed, uint8_t* codes,
                       float* consts, void* stream) {
  return qlora_quantize_nf4_typed(d, W, QLORA_W_F32, packed, codes, consts, stream);
}

int qlora_quantize_nf4_typed(const qlora_nf4_desc* d, const void* W, int32_t w_format, uint8_t* packed,
                             uint8_t* codes, float* consts, void* stream) {
  const int st = check_desc(d);
  if (st) return st;
  if (!W || !packed || (!codes && d->dq_blocksize) || !consts) return QLORA_ERR_NULL;
  static_assert(QLORA_W_F32 == kWeightF32 && QLORA_W_BF16 == kWeightBf16 && QLORA_W_F16 == kWeightF16,
                "weight formats");
  if (w_format != QLORA_W_F32 && w_format != QLORA_W_BF16 && w_format != QLORA_W_F16) return QLORA_ERR_UNSUPPORTED;
  if (!aligned16(W) || !aligned16(packed)) return QLORA_ERR_UNSUPPORTED;
  HIP_TRY(launch_nf4_quantize(W, w_format, packed, codes, consts, d->d_out * d->d_in, d->blocksize,
                              d->dq_blocksize != 0, d->table, (hipStream_t)stream));
  return QLORA_OK;
}

int qlora_dequantize_nf4(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes,
                         const float* consts, uint16_t* W_hat, void* stream) {
  return qlora_merge_lora(d, packed, codes, consts, 0, 0.0f, nullptr, nullptr, W_hat, stream);
}

int qlora_merge_lora(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes,
                     const float* consts, int32_t r, float alpha, const uint16_t* A, const uint16_t* B,
                     uint16_t* W_merged, void* stream) {
  const int st = check_layer(d, 0, r);
  if (st) return st;
  if (!packed || (!codes && d->dq_blocksize) || !consts || !W_merged) return QLORA_ERR_NULL;
  if (r > 0 && (!A || !B)) return QLORA_ERR_NULL;
  if (!aligned16(W_merged) || (r > 0 && (!aligned16(A) || !aligned16(B)))) return QLORA_ERR_UNSUPPORTED;
  const float s = r > 0 ? alpha / (float)r : 0.0f;
  HIP_TRY(launch_export(packed, codes, consts, d->d_out, d->d_in, r, s, A, B, W_merged, d->table, block_shift(d),
                        d->dq_blocksize != 0, (hipStream_t)stream));
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

namespace {
// Everything a forward call checks before it enqueues anything.
static int validate_fwd(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes, const float* consts, int64_t T,
                 const uint16_t* X, int32_t r, const uint16_t* A, const uint16_t* B, const uint16_t* Y,
                 const float* U_out, void* workspace, size_t workspace_bytes, bool check_workspace = true) {
  const int st = check_layer(d, T, r);
  if (st) return st;
  if (!packed || (!codes && d->dq_blocksize) || !consts) return QLORA_ERR_NULL;
  if (T > 0 && (!X || !Y)) return QLORA_ERR_NULL;
  if (r > 0 && (!A || !B)) return QLORA_ERR_NULL;
  if (!aligned16(packed) || !aligned16(X) || !aligned16(A) || !aligned16(B) || !aligned16(Y) || !aligned16(U_out))
    return QLORA_ERR_UNSUPPORTED;
  if (!check_workspace) return QLORA_OK;
  const size_t need = plan_fwd(d, T, r, nullptr).bytes;
  if (need > 0 && (!workspace || workspace_bytes < need)) return QLORA_ERR_WORKSPACE;
  return QLORA_OK;
}

// The launches of a validated forward.  Xa: the adapter's input (X itself,
// or X with dropout applied).
static int enqueue_fwd(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes, const float* consts, int64_t T,
                const uint16_t* X, const uint16_t* Xa, int32_t r, float alpha, const uint16_t* A, const uint16_t* B,
                uint16_t* Y, float* U_out, void* workspace, void* stream) {
  if (T == 0) return QLORA_OK;
  hipStream_t s_ = (hipStream_t)stream;
  FwdWs w = plan_fwd(d, T, r, workspace);
  const int64_t N = d->d_out, K = d->d_in;
  const float s = r > 0 ? alpha / (float)r : 0.0f;
  float* U = U_out ? U_out : w.U;

  if (r > 0) {
    const int e = lora_down(Xa, A, T, K, r, s, w.part, U, w.Us, s_);
    if (e) return e;
  }
  // few tokens: the weight-streaming kernel (it stages 8-bit codes in LDS, so
  // those must be 16-byte aligned; fp32 block scales are loaded per chunk)
  if (T <= kDecodeMaxT && decode_ok(d, codes, consts)) {
    HIP_TRY(launch_decode(packed, codes, consts, X, T, N, K, w.Us, hilo_ld(r), B, r, Y, d->table, block_shift(d),
                          d->dq_blocksize == 0, w.dpart, w.dpart_bytes, s_));
    return QLORA_OK;
  }
  FusedParams fp{};
  fp.A = X; fp.lda = K;
  fp.packed = packed; fp.codes = codes; fp.consts = consts; fp.Kw = K; fp.table = d->table; fp.bshift = block_shift(d);
  fp.dq = d->dq_blocksize != 0;
  fp.M = T; fp.N = N; fp.K0 = K;
  fp.At = w.Us; fp.ldat = hilo_ld(r); fp.Bt = B; fp.ldbt = r; fp.r = r;
  fp.C = Y; fp.ldc = N;
  HIP_TRY(launch_fused(fp, false, s_, KID_FWD_GEMM));
  return QLORA_OK;
}

static int linear_fwd(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes, const float* consts, int64_t T,
               const uint16_t* X, int32_t r, float alpha, const uint16_t* A, const uint16_t* B, uint16_t* Y,
               float* U_out, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = validate_fwd(d, packed, codes, consts, T, X, r, A, B, Y, U_out, workspace, workspace_bytes);
  if (st) return st;
  return enqueue_fwd(d, packed, codes, consts, T, X, X, r, alpha, A, B, Y, U_out, workspace, stream);
}
}  // namespace

int qlora_linear_fwd(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes,
                     const float* consts, int64_t T, const uint16_t* X, int32_t r, float alpha,
                     const uint16_t* A, const uint16_t* B, uint16_t* Y, float* U_out,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return linear_fwd(d, packed, codes, consts, T, X, r, alpha, A, B, Y, U_out, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The forward without a caller workspace: its scratch (U when not saved, the
// hi/lo pairs of s*U, split-contraction partials) lives in a file-scope
// device array.  Each GPU holds its own copy of the array; the host side
// only ever uses the address hipGetSymbolAddress returns for the current
// device, looked up once per device and kept.
// ---------------------------------------------------------------------------

static __device__ __align__(256) unsigned char scratch[QLORA_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of the current device's copy of `scratch`.
int static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QLORA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QLORA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QLORA_OK;
}
}  // namespace

extern "C" {

int qlora_linear_fwd_noalloc(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes,
                             const float* consts, int64_t T, const uint16_t* X, int32_t r, float alpha,
                             const uint16_t* A, const uint16_t* B, uint16_t* Y, float* U_out, void* stream) {
  int st = validate_fwd(d, packed, codes, consts, T, X, r, A, B, Y, U_out, nullptr, 0, false);
  if (st) return st;
  if (plan_fwd(d, T, r, nullptr).bytes > (size_t)QLORA_STATIC_SCRATCH_BYTES) return QLORA_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if ((st = static_scratch(&ws))) return st;
  return enqueue_fwd(d, packed, codes, consts, T, X, X, r, alpha, A, B, Y, U_out, ws, stream);
}

namespace {
// Everything a backward call checks before it enqueues anything.
static int validate_bwd(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes, const float* consts, int64_t T,
                 const uint16_t* X, int32_t r, const uint16_t* A, const uint16_t* B, const float* U_in,
                 const uint16_t* dY, const uint16_t* dX, const float* dA, const float* dB, void* workspace,
                 size_t workspace_bytes) {
  const int st = check_layer(d, T, r);
  if (st) return st;
  if (!packed || (!codes && d->dq_blocksize) || !consts) return QLORA_ERR_NULL;
  if (T > 0 && (!X || !dY)) return QLORA_ERR_NULL;
  if (r > 0 && (!A || !B || !dA || !dB)) return QLORA_ERR_NULL;
  if (!aligned16(packed) || !aligned16(X) || !aligned16(dY) || !aligned16(A) || !aligned16(B) || !aligned16(dX) ||
      !aligned16(U_in) || !aligned16(dA) || !aligned16(dB))
    return QLORA_ERR_UNSUPPORTED;
  const size_t need = plan_bwd(d, T, r, nullptr).bytes;
  if (need > 0 && (!workspace || workspace_bytes < need)) return QLORA_ERR_WORKSPACE;
  return QLORA_OK;
}

// The launches of a validated backward.  Xa: the adapter's input (X, or X
// with dropout applied); keep (optional): the dropout mask, whose factor c
// scales the adapter's share of dX; dx_accumulate: the dX product adds to
// what dX holds.
// Parts of a backward (enqueue_bwd's `phases`): U and G with their hi/lo
// pairs, the dX product, the adapter gradients.
constexpr int kBwdPre = 1, kBwdDx = 2, kBwdGrads = 4, kBwdAll = 7;

static int enqueue_bwd(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes, const float* consts, int64_t T,
                const uint16_t* X, const uint16_t* Xa, const uint8_t* keep, float c, int32_t r, float alpha,
                const uint16_t* A, const uint16_t* B, const float* U_in, const uint16_t* dY, uint16_t* dX, float* dA,
                float* dB, void* workspace, void* stream, int accumulate, int dx_accumulate, int phases = kBwdAll) {
  hipStream_t s_ = (hipStream_t)stream;
  const int64_t N = d->d_out, K = d->d_in;
  if (T == 0) {
    if (r > 0 && !accumulate) {
      HIP_TRY(launch_fill_zero(dA, (int64_t)r * K, s_));
      HIP_TRY(launch_fill_zero(dB, N * r, s_));
    }
    return QLORA_OK;
  }
  BwdWs w = plan_bwd(d, T, r, workspace);
  const float s = r > 0 ? alpha / (float)r : 0.0f;
  const int64_t ldh = hilo_ld(r);

  if (r > 0 && (phases & kBwdPre)) {
    // U = X A^T when the forward's U is not given (its hi/lo pair feeds dB)
    if (!U_in) {
      const int e = lora_down(Xa, A, T, K, r, s, w.part, w.U, w.Us, s_);
      if (e) return e;
    }
    // G = dY B -> hi/lo of s*G (feeds the dX tail and dA); the same launch
    // turns the given U into the hi/lo pair of s*U
    if (lora_rows_ok(T, r)) {
      RowsParams R{};
      R.P = dY; R.ldp = N; R.M = T; R.D = N;
      R.Q = B; R.ldq = r; R.q_strided = 1; R.r = r; R.s = s;
      R.Hout = w.Gs; R.ldh = ldh;
      if (U_in) { R.Uc = U_in; R.Ucs = w.Us; }
      HIP_TRY(launch_lora_rows(R, w.part, w.part_bytes, s_, KID_LORA_G));
    } else {
      SkinnyParams S = skinny(dY, N, true, T, N, r, s, r, OUT_ROWS_HILO, w.part);
      skinny_q(S, B, r, r, Q_STRIDED);
      S.Hout = w.Gs; S.ldh = ldh;
      if (U_in) { S.Uc = U_in; S.Ucs = w.Us; }
      HIP_TRY(launch_skinny(S, s_, KID_LORA_G));
    }
  }
  if (dX && (phases & kBwdDx)) {
    // dX = dY W_hat + (s G) A: the contraction runs over d_out, the rows of W
    FusedParams fp{};
    fp.A = dY; fp.lda = N;
    fp.packed = packed; fp.codes = codes; fp.consts = consts; fp.Kw = K; fp.table = d->table; fp.bshift = block_shift(d);
    fp.dq = d->dq_blocksize != 0;
    fp.M = T; fp.N = K; fp.K0 = N;
    fp.At = w.Gs; fp.ldat = ldh; fp.Bt = A; fp.ldbt = K;
    fp.r = keep ? 0 : r;  // with dropout the adapter's share is added after, through the mask
    fp.C = dX; fp.ldc = K;
    fp.accumulate = dx_accumulate;
    HIP_TRY(launch_fused(fp, true, s_, KID_DX_GEMM));
    if (keep && r > 0) {
      DropoutDxParams Dp{};
      Dp.dX = dX; Dp.Gs = w.Gs; Dp.ldh = ldh; Dp.A = A; Dp.keep = keep; Dp.c = c; Dp.T = T; Dp.K = K; Dp.r = r;
      HIP_TRY(launch_dropout_dx_add(Dp, s_));
    }
  }
  if (r > 0 && (phases & kBwdGrads)) {
    // one launch for both adapter gradients, contractions over the hi/lo columns:
    // dA = (s G)^T X -> [r][d_in]; dB = dY^T (s U) -> [d_out][r]
    if (lora_stream_ok(r)) {
      ColsBatch C{};
      C.p[0] = ColsParams{Xa, K, K, w.Gs, ldh, T, r, 1, dA, accumulate};
      C.p[1] = ColsParams{dY, N, N, w.Us, ldh, T, r, 0, dB, accumulate};
      C.n = 2;
      HIP_TRY(launch_lora_cols(C, w.part, w.part_bytes, s_, KID_LORA_DA));
    } else {
      SkinnyParams Sa = skinny(Xa, K, false, K, T, r, s, 2 * r, OUT_PAIRS_T, w.part);
      skinny_q(Sa, w.Gs, ldh, 2 * (int64_t)r, Q_STRIDED);
      Sa.Fout = dA;
      Sa.accumulate = accumulate;
      SkinnyParams Sb = skinny(dY, N, false, N, T, r, s, 2 * r, OUT_PAIRS, w.part2);
      skinny_q(Sb, w.Us, ldh, 2 * (int64_t)r, Q_STRIDED);
      Sb.Fout = dB;
      Sb.accumulate = accumulate;
      HIP_TRY(launch_skinny_pair(Sa, Sb, s_, KID_LORA_DA));
    }
  }
  return QLORA_OK;
}

static int linear_bwd(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes, const float* consts, int64_t T,
               const uint16_t* X, int32_t r, float alpha, const uint16_t* A, const uint16_t* B, const float* U_in,
               const uint16_t* dY, uint16_t* dX, float* dA, float* dB, void* workspace, size_t workspace_bytes,
               void* stream, int accumulate) {
  const int st = validate_bwd(d, packed, codes, consts, T, X, r, A, B, U_in, dY, dX, dA, dB, workspace,
                              workspace_bytes);
  if (st) return st;
  return enqueue_bwd(d, packed, codes, consts, T, X, X, nullptr, 1.0f, r, alpha, A, B, U_in, dY, dX, dA, dB,
                     workspace, stream, accumulate, 0);
}
}  // namespace

int qlora_linear_bwd(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes,
                     const float* consts, int64_t T, const uint16_t* X, int32_t r, float alpha,
                     const uint16_t* A, const uint16_t* B, const float* U_in, const uint16_t* dY,
                     uint16_t* dX, float* dA, float* dB, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return linear_bwd(d, packed, codes, consts, T, X, r, alpha, A, B, U_in, dY, dX, dA, dB, workspace, workspace_bytes,
                    stream, 0);
}

int qlora_linear_bwd_accumulate(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes,
                                const float* consts, int64_t T, const uint16_t* X, int32_t r, float alpha,
                                const uint16_t* A, const uint16_t* B, const float* U_in, const uint16_t* dY,
                                uint16_t* dX, float* dA, float* dB, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return linear_bwd(d, packed, codes, consts, T, X, r, alpha, A, B, U_in, dY, dX, dA, dB, workspace, workspace_bytes,
                    stream, 1);
}

namespace {
// Several weights that share X: validation, and each weight's workspace slice
// (its plan_fwd bytes, rounded up to 256).
static int check_multi(int32_t n, const qlora_nf4_desc* d, int64_t T, int32_t r) {
  if (!d) return QLORA_ERR_NULL;
  if (n < 1 || n > kDecodeMaxWeights) return QLORA_ERR_SHAPE;
  for (int i = 0; i < n; ++i) {
    const int st = check_layer(&d[i], T, r);
    if (st) return st;
    if (d[i].d_in != d[0].d_in) return QLORA_ERR_SHAPE;
    if (d[i].blocksize != d[0].blocksize || d[i].dq_blocksize != d[0].dq_blocksize) return QLORA_ERR_UNSUPPORTED;
  }
  return QLORA_OK;
}

static size_t multi_slice(const qlora_nf4_desc* d, int64_t T, int32_t r) {
  return (plan_fwd(d, T, r, nullptr).bytes + 255) & ~(size_t)255;
}

// each layer's share of the workspace of a backward over several layers
static size_t bwd_slice(const qlora_nf4_desc* d, int64_t T, int32_t r) { return align256(plan_bwd(d, T, r, nullptr).bytes); }
}  // namespace

int qlora_multi_fwd_workspace_bytes(int32_t n, const qlora_nf4_desc* d, int64_t T, int32_t r, size_t* bytes) {
  if (!bytes) return QLORA_ERR_NULL;
  const int st = check_multi(n, d, T, r);
  if (st) return st;
  size_t b = 0;
  for (int i = 0; i < n; ++i) b += multi_slice(&d[i], T, r);
  *bytes = b;
  return QLORA_OK;
}

int qlora_multi_bwd_workspace_bytes(int32_t n, const qlora_nf4_desc* d, int64_t T, int32_t r, size_t* bytes) {
  if (!bytes) return QLORA_ERR_NULL;
  const int st = check_multi(n, d, T, r);
  if (st) return st;
  size_t b = 0;
  for (int i = 0; i < n; ++i) b += bwd_slice(&d[i], T, r);
  *bytes = b;
  return QLORA_OK;
}

namespace {
static char* ws_at(void* ws, size_t off) { return ws ? static_cast<char*>(ws) + off : nullptr; }
}  // namespace

int qlora_linear_bwd_multi(int32_t n, const qlora_nf4_desc* d, const uint8_t* const* packed,
                           const uint8_t* const* codes, const float* const* consts, int64_t T, const uint16_t* X,
                           int32_t r, float alpha, const uint16_t* const* A, const uint16_t* const* B,
                           const float* const* U_in, const uint16_t* const* dY, uint16_t* dX, float* const* dA,
                           float* const* dB, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_multi(n, d, T, r);
  if (st) return st;
  if (!packed || !codes || !consts || !dY || (r > 0 && (!A || !B || !dA || !dB))) return QLORA_ERR_NULL;
  // every layer is validated, on its slice of the workspace, before the first launch
  size_t need = 0;
  for (int i = 0; i < n; ++i) need += bwd_slice(&d[i], T, r);
  if (need > 0 && (!workspace || workspace_bytes < need)) return QLORA_ERR_WORKSPACE;
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    const size_t sl = bwd_slice(&d[i], T, r);
    st = validate_bwd(&d[i], packed[i], codes[i], consts[i], T, X, r, r > 0 ? A[i] : nullptr,
                      r > 0 ? B[i] : nullptr, U_in ? U_in[i] : nullptr, dY[i], dX, r > 0 ? dA[i] : nullptr,
                      r > 0 ? dB[i] : nullptr, ws_at(workspace, off), sl);
    if (st) return st;
    off += sl;
  }
  auto layer = [&](int i, int phases, int dx_acc) {
    size_t o = 0;
    for (int k = 0; k < i; ++k) o += bwd_slice(&d[k], T, r);
    return enqueue_bwd(&d[i], packed[i], codes[i], consts[i], T, X, X, nullptr, 1.0f, r, alpha,
                       r > 0 ? A[i] : nullptr, r > 0 ? B[i] : nullptr, U_in ? U_in[i] : nullptr, dY[i], dX,
                       r > 0 ? dA[i] : nullptr, r > 0 ? dB[i] : nullptr, ws_at(workspace, o), stream, 0, dx_acc,
                       phases);
  };
  bool same_table = true;
  for (int i = 1; i < n; ++i) same_table = same_table && d[i].table == d[0].table;
  if (n > 1 && T > 0 && dX && same_table) {
    // X's gradient over all the layers in ONE product: their contractions
    // (rows of each weight, against each layer's dY) follow each other, and
    // every layer's rank-r term is a tail of the same accumulation, so dX is
    // summed in fp32 and rounded once
    for (int i = 0; i < n; ++i)
      if ((st = layer(i, kBwdPre, 0))) return st;
    const int64_t K = d[0].d_in, ldh = hilo_ld(r);
    FusedParams fp{};
    off = 0;
    for (int i = 0; i < n; ++i) {
      const BwdWs w = plan_bwd(&d[i], T, r, ws_at(workspace, off));
      off += bwd_slice(&d[i], T, r);
      if (i == 0) {
        fp.A = dY[0]; fp.lda = d[0].d_out;
        fp.packed = packed[0]; fp.codes = codes[0]; fp.consts = consts[0]; fp.Kw = K; fp.table = d[0].table;
        fp.bshift = block_shift(&d[0]); fp.dq = d[0].dq_blocksize != 0;
        fp.M = T; fp.N = K; fp.K0 = d[0].d_out;
        fp.At = w.Gs; fp.ldat = ldh; fp.Bt = r > 0 ? A[0] : nullptr; fp.ldbt = K; fp.r = r;
        fp.C = dX; fp.ldc = K;
      } else {
        fp.seg[i] = FusedSeg{dY[i], d[i].d_out, packed[i], codes[i], consts[i], d[i].d_out, w.Gs, ldh,
                             r > 0 ? A[i] : nullptr, K, dX, K};
      }
    }
    fp.nseg = n;
    HIP_TRY(launch_fused(fp, true, (hipStream_t)stream, KID_DX_GEMM));
    for (int i = 0; i < n; ++i)
      if ((st = layer(i, kBwdGrads, 0))) return st;
    return QLORA_OK;
  }
  // one layer after another on the stream; from the second on, the dX
  // product adds to the dX the earlier ones wrote
  for (int i = 0; i < n; ++i)
    if ((st = layer(i, kBwdAll, i > 0))) return st;
  return QLORA_OK;
}

int qlora_linear_fwd_multi(int32_t n, const qlora_nf4_desc* d, const uint8_t* const* packed,
                           const uint8_t* const* codes, const float* const* consts, int64_t T, const uint16_t* X,
                           int32_t r, float alpha, const uint16_t* const* A, const uint16_t* const* B,
                           uint16_t* const* Y, float* const* U_out, void* workspace, size_t workspace_bytes,
                           void* stream) {
  int st = check_multi(n, d, T, r);
  if (st) return st;
  if (!packed || !codes || !consts || !Y || (r > 0 && (!A || !B))) return QLORA_ERR_NULL;
  // every layer is validated, on its slice of the workspace, before the first launch
  size_t need = 0;
  for (int i = 0; i < n; ++i) need += multi_slice(&d[i], T, r);
  if (need > 0 && (!workspace || workspace_bytes < need)) return QLORA_ERR_WORKSPACE;
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    const size_t sl = multi_slice(&d[i], T, r);
    st = validate_fwd(&d[i], packed[i], codes[i], consts[i], T, X, r, r > 0 ? A[i] : nullptr,
                      r > 0 ? B[i] : nullptr, Y[i], U_out ? U_out[i] : nullptr, ws_at(workspace, off), sl);
    if (st) return st;
    off += sl;
  }
  if (T == 0) return QLORA_OK;

  hipStream_t s_ = (hipStream_t)stream;
  const int64_t K = d[0].d_in;
  bool fused = T <= kDecodeMaxT;
  for (int i = 0; i < n && fused; ++i) fused = decode_ok(&d[i], codes[i], consts[i]);
  if (!fused && n > 1 && T > kDecodeMaxT) {
    // many tokens: each weight's U = X A^T, then one product over all the
    // weights (their output columns side by side), when every weight is
    // whole 256-column tiles and one table serves them all
    bool same_table = true;
    for (int i = 1; i < n; ++i) same_table = same_table && d[i].table == d[0].table;
    FusedParams fp{};
    fp.A = X; fp.lda = K;
    fp.packed = packed[0]; fp.codes = codes[0]; fp.consts = consts[0]; fp.Kw = K; fp.table = d[0].table;
    fp.bshift = block_shift(&d[0]); fp.dq = d[0].dq_blocksize != 0;
    fp.M = T; fp.N = d[0].d_out; fp.K0 = K;
    fp.ldat = hilo_ld(r); fp.Bt = r > 0 ? B[0] : nullptr; fp.ldbt = r; fp.r = r;
    fp.C = Y[0]; fp.ldc = d[0].d_out;
    fp.nseg = n;
    for (int i = 1; i < n; ++i)
      fp.seg[i] = FusedSeg{X, K, packed[i], codes[i], consts[i], d[i].d_out, nullptr, hilo_ld(r),
                           r > 0 ? B[i] : nullptr, r, Y[i], d[i].d_out};
    if (same_table && fused_wide_ok(fp, false)) {
      const float s = r > 0 ? alpha / (float)r : 0.0f;
      off = 0;
      for (int i = 0; i < n; ++i) {
        FwdWs fw = plan_fwd(&d[i], T, r, ws_at(workspace, off));
        off += multi_slice(&d[i], T, r);
        if (r > 0) {
          const int e = lora_down(X, A[i], T, K, r, s, fw.part, U_out && U_out[i] ? U_out[i] : fw.U, fw.Us, s_);
          if (e) return e;
        }
        if (i == 0) fp.At = fw.Us;
        else fp.seg[i].At = fw.Us;
      }
      HIP_TRY(launch_fused(fp, false, s_, KID_FWD_GEMM));
      return QLORA_OK;
    }
  }
  if (!fused) {  // one forward per weight
    off = 0;
    for (int i = 0; i < n; ++i) {
      st = enqueue_fwd(&d[i], packed[i], codes[i], consts[i], T, X, X, r, alpha, r > 0 ? A[i] : nullptr,
                       r > 0 ? B[i] : nullptr, Y[i], U_out ? U_out[i] : nullptr, ws_at(workspace, off), stream);
      if (st) return st;
      off += multi_slice(&d[i], T, r);
    }
    return QLORA_OK;
  }
  // few tokens: each weight's U = X A^T, then one launch over all the weights
  const float s = r > 0 ? alpha / (float)r : 0.0f;
  DecodeWeight w[kDecodeMaxWeights];
  const uint16_t* us[kDecodeMaxWeights];
  off = 0;
  for (int i = 0; i < n; ++i) {
    FwdWs fw = plan_fwd(&d[i], T, r, ws_at(workspace, off));
    off += multi_slice(&d[i], T, r);
    if (r > 0) {
      const int e = lora_down(X, A[i], T, K, r, s, fw.part, U_out && U_out[i] ? U_out[i] : fw.U, fw.Us, s_);
      if (e) return e;
    }
    w[i] = DecodeWeight{packed[i], codes[i], consts[i], d[i].d_out, r > 0 ? B[i] : nullptr, Y[i], d[i].table};
    us[i] = fw.Us;
  }
  HIP_TRY(launch_decode_multi(w, n, X, T, K, us, hilo_ld(r), r, block_shift(&d[0]), d[0].dq_blocksize == 0, s_));
  return QLORA_OK;
}

namespace {
// X with dropout applied, at the start of the workspace; the rest is the
// plain call's workspace
static size_t dropout_xd_bytes(const qlora_nf4_desc* d, int64_t T) { return ((size_t)(T * d->d_in * 2) + 255) & ~(size_t)255; }

static int check_dropout(const qlora_nf4_desc* d, int64_t T, int32_t r, const uint8_t* keep, float p) {
  if (!(p >= 0.0f && p < 1.0f)) return QLORA_ERR_UNSUPPORTED;
  if (T > 0 && r > 0 && !keep) return QLORA_ERR_NULL;
  return QLORA_OK;
}

static float dropout_factor(float p) { return 1.0f / (1.0f - p); }
}  // namespace

int qlora_dropout_workspace_bytes(const qlora_nf4_desc* d, int64_t T, int32_t r, int32_t backward, size_t* bytes) {
  if (!bytes) return QLORA_ERR_NULL;
  const int st = check_layer(d, T, r);
  if (st) return st;
  *bytes = dropout_xd_bytes(d, T) + (backward ? plan_bwd(d, T, r, nullptr).bytes : plan_fwd(d, T, r, nullptr).bytes);
  return QLORA_OK;
}

int qlora_linear_fwd_dropout(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes,
                             const float* consts, int64_t T, const uint16_t* X, int32_t r, float alpha,
                             const uint16_t* A, const uint16_t* B, const uint8_t* keep, float p, uint16_t* Y,
                             float* U_out, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_layer(d, T, r);
  if (st) return st;
  if ((st = check_dropout(d, T, r, keep, p))) return st;
  if (r == 0 || T == 0)
    return linear_fwd(d, packed, codes, consts, T, X, r, alpha, A, B, Y, U_out, workspace, workspace_bytes, stream);
  // X_d at the start of the workspace, the plain call's workspace after it;
  // everything is validated before the first launch
  const size_t xd = dropout_xd_bytes(d, T);
  if (!workspace || workspace_bytes < xd) return QLORA_ERR_WORKSPACE;
  st = validate_fwd(d, packed, codes, consts, T, X, r, A, B, Y, U_out, ws_at(workspace, xd), workspace_bytes - xd);
  if (st) return st;
  uint16_t* Xd = static_cast<uint16_t*>(workspace);
  HIP_TRY(launch_dropout_input(X, keep, dropout_factor(p), T, d->d_in, Xd, (hipStream_t)stream));
  return enqueue_fwd(d, packed, codes, consts, T, X, Xd, r, alpha, A, B, Y, U_out, ws_at(workspace, xd), stream);
}

int qlora_linear_bwd_dropout(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes,
                             const float* consts, int64_t T, const uint16_t* X, int32_t r, float alpha,
                             const uint16_t* A, const uint16_t* B, const float* U_in, const uint16_t* dY,
                             const uint8_t* keep, float p, uint16_t* dX, float* dA, float* dB, int32_t accumulate,
                             void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_layer(d, T, r);
  if (st) return st;
  if ((st = check_dropout(d, T, r, keep, p))) return st;
  if (r == 0 || T == 0)
    return linear_bwd(d, packed, codes, consts, T, X, r, alpha, A, B, U_in, dY, dX, dA, dB, workspace,
                      workspace_bytes, stream, accumulate != 0);
  const size_t xd = dropout_xd_bytes(d, T);
  if (!workspace || workspace_bytes < xd) return QLORA_ERR_WORKSPACE;
  st = validate_bwd(d, packed, codes, consts, T, X, r, A, B, U_in, dY, dX, dA, dB, ws_at(workspace, xd),
                    workspace_bytes - xd);
  if (st) return st;
  uint16_t* Xd = static_cast<uint16_t*>(workspace);
  const float c = dropout_factor(p);
  HIP_TRY(launch_dropout_input(X, keep, c, T, d->d_in, Xd, (hipStream_t)stream));
  return enqueue_bwd(d, packed, codes, consts, T, X, Xd, keep, c, r, alpha, A, B, U_in, dY, dX, dA, dB,
                     ws_at(workspace, xd), stream, accumulate != 0, 0);
}

int qlora_adamw_step(const qlora_adamw_hparams* h, int64_t n, float* param, const float* grad, float* exp_avg,
                     float* exp_avg_sq, uint16_t* param_bf16, void* stream) {
  if (!h) return QLORA_ERR_NULL;
  if (n < 0) return QLORA_ERR_SHAPE;
  const float hp[6] = {h->lr, h->beta1, h->beta2, h->eps, h->weight_decay, h->grad_scale};
  for (float x : hp)
    if (!std::isfinite(x)) return QLORA_ERR_UNSUPPORTED;
  if (h->step < 1 || !(h->beta1 >= 0.0f && h->beta1 < 1.0f) || !(h->beta2 >= 0.0f && h->beta2 < 1.0f) ||
      h->eps < 0.0f)
    return QLORA_ERR_UNSUPPORTED;
  if (n == 0) return QLORA_OK;
  if (!param || !grad || !exp_avg || !exp_avg_sq) return QLORA_ERR_NULL;
  if (!aligned16(param) || !aligned16(grad) || !aligned16(exp_avg) || !aligned16(exp_avg_sq) ||
      (param_bf16 && ((uintptr_t)param_bf16 & 7) != 0))
    return QLORA_ERR_UNSUPPORTED;
  const double t = (double)h->step;
  const double bc1 = 1.0 - std::pow((double)h->beta1, t), bc2 = 1.0 - std::pow((double)h->beta2, t);
  AdamwParams P{};
  P.p = param; P.g = grad; P.m = exp_avg; P.v = exp_avg_sq; P.p16 = param_bf16; P.n = n;
  P.decay = (float)(1.0 - (double)h->lr * (double)h->weight_decay);
  P.gscale = h->grad_scale;
  P.beta1 = h->beta1; P.one_minus_beta1 = (float)(1.0 - (double)h->beta1);
  P.beta2 = h->beta2; P.one_minus_beta2 = (float)(1.0 - (double)h->beta2);
  P.step_size = (float)((double)h->lr / bc1);
  P.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
  P.eps = h->eps;
  HIP_TRY(launch_adamw(P, (hipStream_t)stream));
  return QLORA_OK;
}

}  // extern "C"
