/*
 * qlora.h -- C ABI of the MI355X (gfx950) QLoRA linear-layer library.
 *
 * The layer: a frozen weight W (d_out x d_in) stored as blockwise NF4 with
 * double-quantized scales, plus a trainable rank-r adapter (A, B):
 *     forward   Y  = X W_hat^T + s (X A^T) B^T,          s = fl32(alpha / r)
 *     backward  dX = dY W_hat + s (dY B) A,  dA = s (dY B)^T X,  dB = s dY^T (X A^T)
 * where W_hat is the restored (dequantized, bf16) weight and no gradient is
 * ever formed for W.
 *
 * Sources (page titles and sections):
 *   "QLoRA技术从入门到精通" §2(3) NF4 grid; §3(1) offline quantization
 *       (blocks, absmax scale, normalize, nearest level, 4-bit index, 8-bit
 *       quantization of the scales); §3(2) forward (restore to 16 bit, two
 *       branches, alpha / r); §3(3) backward (frozen base, only A and B).
 *   "LoRA 与 QLoRA：把大模型微调拆成可负担的工程" §2 (h = W x + (alpha/r) B A x,
 *       shapes of A and B), §8 (bf16 compute, bias none).
 *   "【X 长文】LoRA 与 QLoRA：用一块 GPU 微调大模型", quantization section
 *       (64-value blocks, NF4 levels with an exact 0, about 4.13 bits per
 *       weight with 8-bit scales) and QLoRA section (gradient passes through
 *       the restored weight to A and B).
 *   "7、QLoRA 量化微调" §7.1 (16 ascending level indices; group storage).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All matrices are dense and row-major.  bf16 tensors cross the ABI as
 *   uint16_t bit patterns.  Shapes (T = tokens, K = d_in, N = d_out):
 *     W [N][K] fp32, X [T][K], Y [T][N], A [r][K], B [N][r], dY [T][N],
 *     dX [T][K] (bf16); U [T][r], dA [r][K], dB [N][r] (fp32).
 * - Stored weight format (written by qlora_quantize_nf4):
 *     packed [N][K/2] uint8: 4-bit level indices, element 2j of the flattened
 *            weight in the HIGH nibble of byte j, element 2j+1 in the low one;
 *     codes  [N*K/bs] uint8: 8-bit code of each block's absmax scale, a block
 *            being bs consecutive weights of the flattened weight (bs =
 *            desc.blocksize: 64, 128 or 256; blocks may span rows);
 *     consts [ceil(N*K/bs/256)] fp32: per group of 256 consecutive block
 *            scales, the group's largest scale c_g.
 *   Block b is restored with s'_b = fl32(fl32(code_b) * fl32(c_g / 255)) and
 *   each weight as bf16_rne(fl32(T[q] * s'_b)).  With dq_blocksize == 0 there
 *   are no codes: consts [N*K/bs] holds each block's fp32 absmax s_b, and
 *   s'_b = s_b.
 * - Device pointers: every tensor argument is device memory owned by the
 *   caller (the library never allocates, frees or retains device memory and
 *   keeps no state between calls).  Descriptors and output-size pointers are
 *   host memory.
 * - stream: a hipStream_t passed as void* (NULL = the null stream).  Every
 *   compute call only enqueues work on that stream and returns without
 *   synchronizing; outputs are valid once the stream has reached that point.
 * - Errors: functions return QLORA_OK (0) or a negative QLORA_ERR_* code.
 *   Arguments are validated on the host before anything is enqueued -- for
 *   the calls on several layers, every layer before the first launch -- so a
 *   call that fails validation has no side effect.  QLORA_ERR_HIP reports a
 *   failed launch (hipGetLastError after enqueueing); work enqueued before
 *   it by the same call may then have run.
 * - Size limit: the kernels address each dense operand with 32-bit byte
 *   offsets, so the packed weight (N*K/2 bytes), X (T*K*2), Y and dY (T*N*2),
 *   dX (T*K*2) and the [T][2r] rank-r pairs of the workspace must each be
 *   below 2^31 - 16 bytes; larger calls return QLORA_ERR_SHAPE (the workspace
 *   queries too).  Dimensions are below 2^31.
 * - W, packed, X, dY, A, B, Y, dX, U_out, U_in, dA and dB must be 16-byte
 *   aligned (QLORA_ERR_UNSUPPORTED otherwise); codes and consts need only
 *   their element alignment.  A forward
 *   call with at most 16 tokens takes the weight-streaming kernel when K is
 *   a multiple of the block size and either codes is 16-byte aligned and
 *   K/bs is at most about 2000 (8-bit codes), or consts is 16-byte aligned
 *   and K/bs is at most about 1000 (fp32 block scales, dq_blocksize 0); else
 *   the tiled kernel (same results within the accuracy stated below).
 * - Inputs must be finite; results for NaN/Inf inputs are unspecified.
 * - Hot-path preconditions: blocksize 64 (also 128 or 256), dq_blocksize 256 (also 0),
 *   d_in % 64 == 0, d_out % 64 == 0, 0 <= r <= 128, T >= 0 (T == 0 is a
 *   no-op).  r == 0 means the base branch only.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  QLORA_OK = 0,
  QLORA_ERR_NULL = -1,        /* a required pointer is NULL */
  QLORA_ERR_SHAPE = -2,       /* a size is out of range or not a multiple it must be */
  QLORA_ERR_UNSUPPORTED = -3, /* a format parameter the library does not implement */
  QLORA_ERR_WORKSPACE = -4,   /* workspace is NULL or smaller than the size query returned */
  QLORA_ERR_HIP = -5,         /* the HIP runtime reported an error while enqueueing */
  QLORA_ERR_SCRATCH_LIMIT = -6 /* the call needs more scratch than QLORA_STATIC_SCRATCH_BYTES */
};

/* Descriptor of the stored base weight. */
typedef struct qlora_nf4_desc {
  int64_t d_out;        /* N: rows of W */
  int64_t d_in;         /* K: columns of W */
  int32_t blocksize;    /* weights per absmax block: 64, 128 or 256 ("QLoRA技术从入门到精通"
                           §3(1): blocks of e.g. 64 or 256 values) */
  int32_t dq_blocksize; /* block scales per second-level group: 256, or 0 for no second level
                           (the fp32 block scales are kept: consts holds one per block, codes is
                           empty and may be NULL; "7、QLoRA 量化微调" §7.1, 4.5 bits per weight) */
  int32_t table;        /* level table: QLORA_TABLE_NF4 (0) or QLORA_TABLE_UNIFORM (1) */
} qlora_nf4_desc;

/*
 * Level tables.  QLORA_TABLE_NF4: the NF4 table (qlora_nf4_levels).
 * QLORA_TABLE_UNIFORM: 16 equally spaced levels -1 + 2i/15 on [-1, 1]
 * ("7、QLoRA 量化微调" §7.1, with its worked example: 0.27 in a group of
 * absmax 1.52 -> index 9 -> 0.304); it has no zero level.  Everything else
 * (blocks, scale codes, packing, kernels) is the same.  The table is not
 * stored with the quantized weight: every call on a weight must pass the desc
 * it was quantized with.  Any other value: QLORA_ERR_UNSUPPORTED.
 */
#define QLORA_TABLE_NF4 0
#define QLORA_TABLE_UNIFORM 1

/* Human-readable name of a status code.  Never NULL; static storage. */
const char* qlora_status_string(int status);

/*
 * The library's NF4 level table and decision thresholds (host copy).
 * levels[16]: ascending, levels[0] = -1, levels[7] = 0, levels[15] = +1; the
 *   medians of 7 equal-probability slices of the lower half of N(0,1) and of
 *   8 slices of the upper half, each half scaled by its largest magnitude
 *   ("QLoRA技术从入门到精通" §2(3); "【X 长文】..." NF4 paragraph).
 * thresholds[15]: thresholds[k] is the largest float32 that is not closer to
 *   levels[k+1] than to levels[k]; the index of a normalized value x is the
 *   number of thresholds it exceeds (nearest level, ties to the lower index).
 * Either pointer may be NULL.  Host only; never touches the GPU.
 */
int qlora_nf4_levels(float* levels, float* thresholds);

/*
 * The same for either level table (QLORA_TABLE_NF4 or QLORA_TABLE_UNIFORM);
 * the thresholds follow the same rule.  Errors: UNSUPPORTED for another table.
 */
int qlora_table_levels(int32_t table, float* levels, float* thresholds);

/*
 * Sizes in bytes of the three stored-weight buffers for descriptor d.
 * Host only.  Errors: NULL (d or any out pointer), SHAPE, UNSUPPORTED.
 */
int qlora_nf4_sizes(const qlora_nf4_desc* d, size_t* packed_bytes, size_t* codes_bytes,
                    size_t* consts_bytes);

/*
 * Offline quantization of W (fp32 [N][K], device) into packed / codes /
 * consts (device, sizes from qlora_nf4_sizes) -- "QLoRA技术从入门到精通" §3(1):
 * per block (desc.blocksize weights) absmax scale s_b, x = fl32(w / s_b) (IEEE division),
 * nearest NF4 level (ties to the lower index; an all-zero block gives index 7),
 * two indices per byte; then per group of 256 block scales c_g = max s_b and
 * code_b = rint_half_even(fl32(fl32(s_b / c_g) * 255)) (0 when c_g == 0).
 * Indices use the exact s_b.  Results are bit-exact and deterministic.
 * Errors: NULL, SHAPE, UNSUPPORTED, HIP.
 */
int qlora_quantize_nf4(const qlora_nf4_desc* d, const float* W, uint8_t* packed, uint8_t* codes,
                       float* consts, void* stream);

/*
 * The same quantization of a base weight held in a 16-bit format
 * ("QLoRA技术从入门到精通" §3(1): the FP16 base model is converted offline to
 * the 4-bit form).  w_format: QLORA_W_F32 (W is float*, the call above),
 * QLORA_W_BF16 or QLORA_W_F16 (W is [N][K] uint16 bit patterns).  Each value
 * is widened exactly to fp32 and then quantized as above, so the outputs are
 * bit-identical to qlora_quantize_nf4 on the widened weight.  W and packed
 * 16-byte aligned.  Errors: NULL, SHAPE, UNSUPPORTED (unknown w_format,
 * alignment), HIP.
 */
#define QLORA_W_F32 0
#define QLORA_W_BF16 1
#define QLORA_W_F16 2
int qlora_quantize_nf4_typed(const qlora_nf4_desc* d, const void* W, int32_t w_format, uint8_t* packed,
                             uint8_t* codes, float* consts, void* stream);

/*
 * Workspace (device bytes) qlora_linear_fwd needs for T tokens and rank r.
 * Host only.  Errors: NULL, SHAPE, UNSUPPORTED.
 */
int qlora_fwd_workspace_bytes(const qlora_nf4_desc* d, int64_t T, int32_t r, size_t* bytes);

/*
 * Forward of the layer -- "QLoRA技术从入门到精通" §3(2); "LoRA 与 QLoRA：..." §2:
 *   U = X A^T (fp32 [T][r]),  Y = bf16( X W_hat^T + s U B^T ),  s = fl32(alpha/r).
 * W_hat is restored tile by tile on chip and never written to memory.
 * X [T][K], A [r][K], B [N][r], Y [T][N] are bf16 bits (device).  U_out
 * (fp32 [T][r], device) receives U for the backward pass; may be NULL.
 * A and B may be NULL only when r == 0; X and Y only when T == 0.
 * workspace: device scratch of at
 * least qlora_fwd_workspace_bytes (may be NULL if that size is 0); its
 * contents on entry are ignored.  Y must not alias any input.
 * Accuracy: fp32 accumulation of bf16 products; deterministic (no atomics).
 * Errors: NULL, SHAPE, UNSUPPORTED, WORKSPACE, HIP.
 */
int qlora_linear_fwd(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes,
                     const float* consts, int64_t T, const uint16_t* X, int32_t r, float alpha,
                     const uint16_t* A, const uint16_t* B, uint16_t* Y, float* U_out,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * The forward above for callers that cannot allocate device memory -- code
 * recorded into a HIP graph, serving loops, harnesses that forbid hipMalloc:
 * the same kernels and the same results, bit for bit, as qlora_linear_fwd,
 * with no workspace argument.  The scratch comes from a device array of
 * QLORA_STATIC_SCRATCH_BYTES inside the library, one per GPU, kept until the
 * process ends; the call itself allocates and frees nothing.  A call whose
 * scratch (qlora_fwd_workspace_bytes) exceeds it returns
 * QLORA_ERR_SCRATCH_LIMIT before anything is enqueued (at r = 64: above
 * 32768 tokens).  All calls on one GPU share that GPU's array: two calls
 * that may run at the same time on one GPU (other streams, other host
 * threads) race on it and must be ordered by the caller.  The array's
 * contents on entry are ignored.  The stream must belong to the current
 * device (the array's address is looked up for it).  Other arguments,
 * accuracy and errors as qlora_linear_fwd; also HIP when the array cannot be
 * located.
 */
#define QLORA_STATIC_SCRATCH_BYTES (16u << 20)
int qlora_linear_fwd_noalloc(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes,
                             const float* consts, int64_t T, const uint16_t* X, int32_t r, float alpha,
                             const uint16_t* A, const uint16_t* B, uint16_t* Y, float* U_out, void* stream);

/*
 * Workspace (device bytes) qlora_linear_bwd needs for T tokens and rank r.
 * Host only.  Errors: NULL, SHAPE, UNSUPPORTED.
 */
int qlora_bwd_workspace_bytes(const qlora_nf4_desc* d, int64_t T, int32_t r, size_t* bytes);

/*
 * Backward of the layer -- "QLoRA技术从入门到精通" §3(3); "【X 长文】..." QLoRA
 * section (the gradient reaches A and B through the restored weight; the base
 * weight is frozen, so no dW exists):
 *   G  = dY B
 *   dX = bf16( dY W_hat + s G A )        (skipped when dX == NULL)
 *   dA = s G^T X        fp32 [r][K], overwritten (not accumulated)
 *   dB = s dY^T U       fp32 [N][r], overwritten (not accumulated)
 * U_in: fp32 [T][r] saved by the forward; NULL recomputes U = X A^T.
 * dA and dB are required when r > 0 and ignored when r == 0; X and dY may
 * be NULL only when T == 0 (then dA and dB are set to zero).
 * workspace: at least qlora_bwd_workspace_bytes.  Outputs must not alias inputs.
 * Deterministic (no atomics).  Errors: NULL, SHAPE, UNSUPPORTED, WORKSPACE, HIP.
 */
int qlora_linear_bwd(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes,
                     const float* consts, int64_t T, const uint16_t* X, int32_t r, float alpha,
                     const uint16_t* A, const uint16_t* B, const float* U_in, const uint16_t* dY,
                     uint16_t* dX, float* dA, float* dB, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * The backward above for gradient accumulation over micro-batches ("LoRA 与
 * QLoRA：..." §10: gradient accumulation simulates a larger effective batch):
 * identical, except that the adapter gradients are added to what dA and dB
 * hold on entry,
 *   dA += s G^T X,   dB += s dY^T U,
 * each element read, added once in fp32 and written (deterministic; the sum
 * over the micro-batch is formed first, then added).  T == 0 leaves dA and dB
 * unchanged.  dX is written as by qlora_linear_bwd.  Same errors.
 */
int qlora_linear_bwd_accumulate(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes,
                                const float* consts, int64_t T, const uint16_t* X, int32_t r, float alpha,
                                const uint16_t* A, const uint16_t* B, const float* U_in, const uint16_t* dY,
                                uint16_t* dX, float* dA, float* dB, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * Export of the restored weight -- "QLoRA技术从入门到精通" §3(2) (the 4-bit
 * weight restored to a 16-bit float, table value times the block's scale):
 *   W_hat[N][K] = bf16_rne(fl32(T[q] * s'))   (bf16 bits, device)
 * Bit-identical to the weight the fused products restore on chip.  packed,
 * codes, consts as produced by qlora_quantize_nf4; W_hat must be 16-byte
 * aligned and must not alias the inputs.
 * Errors: NULL, SHAPE, UNSUPPORTED, HIP.
 */
int qlora_dequantize_nf4(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes,
                         const float* consts, uint16_t* W_hat, void* stream);

/*
 * The adapter merged into the restored weight -- "LoRA 与 QLoRA：把大模型微调拆成
 * 可负担的工程" §3 (W + (alpha/r) B A after training); "【X 长文】LoRA 与 QLoRA：
 * 用一块 GPU 微调大模型", QLoRA section (with a 4-bit base, the merge goes into
 * the restored 16-bit weight, not into the 4-bit one):
 *   W_merged[N][K] = bf16_rne( fl32( W_hat + fl32(s * (B A)) ) ),  s = fl32(alpha / r)
 * A [r][K] and B [N][r] are bf16 bits (device, 16-byte aligned); B A is
 * accumulated in fp32 (MFMA order).  r = 0 gives W_hat exactly.  1 <= r <= 128
 * otherwise.  The 4-bit arrays are not modified.
 * Errors: NULL, SHAPE, UNSUPPORTED, HIP.
 */
int qlora_merge_lora(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes,
                     const float* consts, int32_t r, float alpha, const uint16_t* A, const uint16_t* B,
                     uint16_t* W_merged, void* stream);

/*
 * Forward of n (1..4) layers that share their input X -- the projections of
 * one layer input, e.g. the query, key and value projections or the gate and
 * up projections; "LoRA 与 QLoRA：..." §8 targets every linear module, so
 * these arrive together.  Each layer i is the forward of qlora_linear_fwd
 * with d[i], packed[i], codes[i], consts[i], A[i], B[i], Y[i] and U_out[i];
 * all share X, T, r and alpha.  The layers must have the same d_in,
 * blocksize and dq_blocksize (tables may differ).  With at most 16 tokens the
 * rows of every weight are streamed in ONE launch (one workgroup per group of
 * row tiles, whichever weight they belong to), so small projections do not
 * leave the GPU idle and X is read from HBM once.  With more tokens, when
 * n > 1, every d_out is a multiple of 256, all layers use one table and the
 * weights' 256 x 256 output tiles number 512 or more, each layer's U runs
 * first and then ONE product covers all the weights (their output columns
 * side by side, each tile writing into its own layer's Y); otherwise the
 * layers run one after another.  Either way each Y element is the same
 * fp32 sum, rounded once.  The pointer arrays are host memory holding device
 * pointers; U_out may be NULL, or hold NULL entries.  Workspace:
 * qlora_multi_fwd_workspace_bytes.  Errors: as qlora_linear_fwd, and SHAPE
 * (n outside 1..4, different d_in), UNSUPPORTED (different block format).
 */
int qlora_multi_fwd_workspace_bytes(int32_t n, const qlora_nf4_desc* d, int64_t T, int32_t r, size_t* bytes);
int qlora_linear_fwd_multi(int32_t n, const qlora_nf4_desc* d, const uint8_t* const* packed,
                           const uint8_t* const* codes, const float* const* consts, int64_t T, const uint16_t* X,
                           int32_t r, float alpha, const uint16_t* const* A, const uint16_t* const* B,
                           uint16_t* const* Y, float* const* U_out, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Backward of n (1..4) layers that share their input X (as for
 * qlora_linear_fwd_multi): X's gradient is the sum of the layers' shares,
 *   dX = bf16( sum_i (dY_i W_hat_i + s G_i A_i) ).
 * When n > 1, T > 0, dX is given and all layers use one table, dX is ONE
 * product: its contraction runs over the rows of every weight in turn (each
 * against its layer's dY), then over every layer's rank-r term, all in one
 * fp32 sum per element, rounded once.  Otherwise it is formed layer after
 * layer: the first layer's product writes dX, and each later one rounds its
 * own share to bf16, adds it to what dX holds and rounds again.  dA[i] and
 * dB[i] are each layer's own, overwritten.  U_in may be NULL or hold NULL
 * entries (U recomputed).  dX may be NULL.  Each layer has its own slice of
 * the workspace (qlora_multi_bwd_workspace_bytes is the sum of the slices).
 * Errors: as qlora_linear_bwd, and SHAPE (n outside 1..4, different d_in),
 * UNSUPPORTED (different block format).
 */
int qlora_multi_bwd_workspace_bytes(int32_t n, const qlora_nf4_desc* d, int64_t T, int32_t r, size_t* bytes);
int qlora_linear_bwd_multi(int32_t n, const qlora_nf4_desc* d, const uint8_t* const* packed,
                           const uint8_t* const* codes, const float* const* consts, int64_t T, const uint16_t* X,
                           int32_t r, float alpha, const uint16_t* const* A, const uint16_t* const* B,
                           const float* const* U_in, const uint16_t* const* dY, uint16_t* dX, float* const* dA,
                           float* const* dB, void* workspace, size_t workspace_bytes, void* stream);

/*
 * LoRA dropout on the adapter's input ("LoRA 与 QLoRA：..." §4.3; its §8
 * configuration uses lora_dropout 0.05).  The base branch takes X unchanged;
 * the adapter takes X_d = bf16_rne(fl32(x * c)) where kept and 0 where
 * dropped, c = fl32(1 / fl32(1 - p)):
 *   forward   U = X_d A^T,  Y = bf16(X W_hat^T + s U B^T)
 *   backward  dX = bf16(bf16(dY W_hat) + keep * c * (s G A)),  dA = s G^T X_d,
 *             dB = s dY^T U          (G = dY B; U as saved by the forward)
 * keep: the mask, an input (the random draw is the caller's): device,
 * [T][K/8] bytes, bit j of byte i (least significant first) keeps element
 * 8i + j of the row.  p in [0, 1).  The adapter's share of dX is added to the
 * rounded base share, so dX is rounded twice (once more than without
 * dropout).  Workspace: qlora_dropout_workspace_bytes (backward = 0 or 1);
 * its first T*K*2 bytes (rounded up to 256) hold X_d.  accumulate != 0 adds
 * to dA and dB as qlora_linear_bwd_accumulate does.  Other arguments as in
 * qlora_linear_fwd / qlora_linear_bwd.  r == 0 or T == 0: the plain call.
 * Errors: as those calls, and NULL (keep when T > 0 and r > 0),
 * UNSUPPORTED (p outside [0, 1)).
 */
int qlora_dropout_workspace_bytes(const qlora_nf4_desc* d, int64_t T, int32_t r, int32_t backward, size_t* bytes);
int qlora_linear_fwd_dropout(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes,
                             const float* consts, int64_t T, const uint16_t* X, int32_t r, float alpha,
                             const uint16_t* A, const uint16_t* B, const uint8_t* keep, float p, uint16_t* Y,
                             float* U_out, void* workspace, size_t workspace_bytes, void* stream);
int qlora_linear_bwd_dropout(const qlora_nf4_desc* d, const uint8_t* packed, const uint8_t* codes,
                             const float* consts, int64_t T, const uint16_t* X, int32_t r, float alpha,
                             const uint16_t* A, const uint16_t* B, const float* U_in, const uint16_t* dY,
                             const uint8_t* keep, float p, uint16_t* dX, float* dA, float* dB, int32_t accumulate,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * AdamW update of the adapter parameters ("QLoRA技术从入门到精通" §3(3):
 * after the backward pass the optimizer updates only A and B, never the
 * quantized base weight).  The arithmetic is the published AdamW method
 * (Loshchilov and Hutter, decoupled weight decay), per element in fp32 with
 * the fp32 hyperparameters as given; the factors below that depend on them
 * (1 - beta, 1 - lr * weight_decay, the bias corrections) are formed in double
 * on the host and rounded to fp32 once:
 *   g = grad * grad_scale;  p *= 1 - lr * weight_decay
 *   m = beta1 m + (1 - beta1) g;  v = beta2 v + (1 - beta2) g^2
 *   p -= (lr / (1 - beta1^step)) * m / (sqrt(v) / sqrt(1 - beta2^step) + eps)
 *   param_bf16 = bf16_rne(p)        (skipped when param_bf16 == NULL)
 * param, grad, exp_avg (m), exp_avg_sq (v): fp32 [n], device, 16-byte
 * aligned, updated in place (grad is read only); param_bf16: uint16 [n]
 * bf16 bits, 8-byte aligned.  Lay out every adapter of a model in one arena
 * to update them all in one call; with gradient accumulation, grad_scale =
 * 1 / (number of micro-batches) averages them.  The paged placement of the
 * optimizer state is not part of this call.  No buffer may alias another.
 * n == 0 does nothing (the buffers may then be NULL).
 * Errors: NULL (h; param, grad, exp_avg or exp_avg_sq when n > 0), SHAPE (n < 0),
 * UNSUPPORTED (step < 1, beta outside [0, 1), eps < 0, non-finite
 * hyperparameters, alignment), HIP.
 */
typedef struct qlora_adamw_hparams {
  float lr;
  float beta1;
  float beta2;
  float eps;
  float weight_decay;
  float grad_scale;
  int64_t step;  /* 1 for the first update */
} qlora_adamw_hparams;

int qlora_adamw_step(const qlora_adamw_hparams* h, int64_t n, float* param, const float* grad, float* exp_avg,
                     float* exp_avg_sq, uint16_t* param_bf16, void* stream);

/*
 * Per-kernel timing (measurement support; not an operation of the layer).
 * qlora_trace_enable(1) makes every subsequent kernel launch of the library
 * record a hipEvent before and after it on the launch stream (event objects
 * are created on first use and reused; no device memory is allocated);
 * qlora_trace_enable(0) (the default) records nothing.
 * qlora_trace_read waits for the recorded events, adds their elapsed times to
 * per-kernel totals and writes up to max_stats entries {name, launches,
 * total_ms} (name: static string) for the kernels launched so far; *count
 * receives the number of kernels with launches.  reset != 0 clears the
 * totals afterwards.  Errors: NULL (count, or stats with max_stats > 0), HIP.
 * Not thread-safe with respect to concurrent compute calls on other threads.
 */
/*
 * qlora_trace_select: like qlora_trace_enable, but only the kernels whose bit
 * is set in kernel_mask are bracketed (bit k = the kernel named by
 * qlora_trace_kernel_name(k)), so a caller can time the big kernels without
 * adding events between all the small ones.  qlora_trace_kernel_name returns
 * a static name, or NULL for k outside the library's kernel list.
 */
int qlora_trace_select(uint32_t kernel_mask);
const char* qlora_trace_kernel_name(int kernel);

typedef struct qlora_kernel_stat {
  const char* name;
  int64_t launches;
  double total_ms;
} qlora_kernel_stat;

int qlora_trace_enable(int enable);
int qlora_trace_read(qlora_kernel_stat* stats, int max_stats, int* count, int reset);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H */
