"""QLoRA linear layer forward/backward -- CPU oracle (float64).

TEST INFRASTRUCTURE ONLY (see ``oracle``): never imported by the product path.

What it follows:

* Forward, two branches ([QLoRA-入门到精通] §3(2); [LoRA-QLoRA-工程] §2):
  the base branch multiplies the restored (dequantized, bf16) weight with the
  input, the LoRA branch multiplies by A (r x d_in) then B (d_out x r), and the
  branches are summed with the LoRA branch scaled by alpha / r.  In the
  row-token convention used here (X is [T][d_in], one token per row):
      U = X A^T,    Y = X W^T + s * U B^T,    s = fl32(alpha / r).
  Reading for evaluation order (pages silent; [QLoRA-入门到精通] writes
  (B A) x, [X长文] "pattern" section describes a rank-1 pattern reading its
  input direction first): both orders are equal in exact arithmetic; the
  oracle evaluates B (A x), and ``merged_weight`` gives the (W + s B A) form.
* Backward ([QLoRA-入门到精通] §3(3); [X长文] QLoRA section): the base weight
  is frozen (no gradient is formed for it), the gradient flows through the
  restored weight to the earlier layer and into A and B.  By the chain rule:
      G  = dY B
      dX = dY W + s * G A
      dA = s * G^T X
      dB = s * dY^T U
  No bias on this path ([LoRA-QLoRA-工程] §8 configuration has bias
  "none"); LoRA dropout, a separate option, is ``forward_dropout`` /
  ``backward_dropout`` below.

All arithmetic is float64 from the exact bf16 input values.  Matrix products
use numpy's matmul (a library primitive).

Pins (``tests/test_oracle_lora.py``): the rank-1 and rank-2 sales tables of
[X长文] "pattern" section through the layer (exact), B = 0 reproduces the base
path exactly and leaves dA = 0 ([LoRA-QLoRA-工程] §3; [X长文] LoRA section),
merge equivalence ([LoRA-QLoRA-工程] §3; [X长文] QLoRA section), central finite
differences of ``forward`` and torch.autograd in float64 for ``backward``.
"""

import numpy as np


def lora_scale(alpha: float, r: int) -> float:
    """s = alpha / r, rounded to float32 (the scalar the layer multiplies by)."""
    if r == 0:
        return 0.0
    return float(np.float32(alpha) / np.float32(r))


def forward(W_hat, X, A, B, alpha: float, r: int):
    """Y = X W_hat^T + s (X A^T) B^T; returns (Y, U) in float64.

    ``W_hat`` [d_out][d_in] is the restored weight (``nf4.dequantize``),
    ``X`` [T][d_in], ``A`` [r][d_in], ``B`` [d_out][r] are float arrays of the
    exact bf16 values.  ``r == 0`` means the base branch only.
    """
    W_hat = np.asarray(W_hat, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    base = X @ W_hat.T
    if r == 0:
        return base, np.zeros((X.shape[0], 0))
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    s = lora_scale(alpha, r)
    U = X @ A.T
    Y = base + s * (U @ B.T)
    return Y, U


def backward(W_hat, X, A, B, dY, alpha: float, r: int):
    """Gradients of the layer for upstream gradient dY [T][d_out].

    Returns (dX [T][d_in], dA [r][d_in], dB [d_out][r]) in float64; there is
    no gradient for the frozen base weight.
    """
    W_hat = np.asarray(W_hat, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    dY = np.asarray(dY, dtype=np.float64)
    dX = dY @ W_hat
    if r == 0:
        return dX, np.zeros((0, X.shape[1])), np.zeros((W_hat.shape[0], 0))
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    s = lora_scale(alpha, r)
    G = dY @ B
    U = X @ A.T
    dX = dX + s * (G @ A)
    dA = s * (G.T @ X)
    dB = s * (dY.T @ U)
    return dX, dA, dB


def merged_weight(W_hat, A, B, alpha: float, r: int) -> np.ndarray:
    """W_hat + s B A in float64: the adapter merged into the restored 16-bit
    weight, never into the 4-bit one ([LoRA-QLoRA-工程] §3; [X长文] QLoRA
    section, cost paragraph)."""
    W_hat = np.asarray(W_hat, dtype=np.float64)
    if r == 0:
        return W_hat.copy()
    return W_hat + lora_scale(alpha, r) * (np.asarray(B, np.float64) @ np.asarray(A, np.float64))


# ----------------------------------------------------------------------------
# LoRA dropout on the adapter's input
# ----------------------------------------------------------------------------
#
# [LoRA-QLoRA-工程] §4.3: LoRA dropout randomly drops elements of the adapter's
# input (its §8 configuration uses lora_dropout = 0.05); the base branch sees
# the undropped input.  Reading (the pages give no arithmetic): inverted
# dropout, the usual form, in the layer's 16-bit compute type --
#     X_d = bf16_rne(fl32(X * c)) where kept, 0 where dropped,  c = fl32(1 / (1 - p))
#     U = X_d A^T,   Y = X W^T + s U B^T.
# The mask is an input (the random draw is not part of the layer): keep bits,
# row t holding d_in / 8 bytes, bit j of byte i (least significant first)
# keeping element 8 i + j.  By the chain rule the adapter's share of dX passes
# back through the same mask and factor:
#     dX = dY W + (s G A) * keep * c,   dA = s G^T X_d,   dB = s dY^T U.


def unpack_keep(keep_bits, d_in: int) -> np.ndarray:
    """[T][d_in / 8] uint8 keep bits -> [T][d_in] bool (bit j of byte i keeps 8i + j)."""
    b = np.asarray(keep_bits, dtype=np.uint8)
    return np.unpackbits(b, axis=1, bitorder="little")[:, :d_in].astype(bool)


def dropout_factor(p: float) -> float:
    """c = fl32(1 / (1 - p)), the factor kept elements are multiplied by."""
    return float(np.float32(1.0) / (np.float32(1.0) - np.float32(p)))


def dropped_input(X, keep_bits, p: float, round_bf16: bool = True) -> np.ndarray:
    """X_d: kept elements times c (rounded to bf16 unless round_bf16 is False),
    dropped elements 0; float64."""
    from .bf16 import round_to_bf16
    X = np.asarray(X, dtype=np.float64)
    keep = unpack_keep(keep_bits, X.shape[1])
    c = dropout_factor(p)
    v = X * c
    if round_bf16:
        v = round_to_bf16(v.astype(np.float32)).astype(np.float64)   # fl32(X * c), then bf16
    return np.where(keep, v, 0.0)


def forward_dropout(W_hat, X, A, B, alpha: float, r: int, keep_bits, p: float, round_bf16: bool = True):
    """Y = X W^T + s (X_d A^T) B^T; returns (Y, U) in float64."""
    W_hat = np.asarray(W_hat, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    Xd = dropped_input(X, keep_bits, p, round_bf16)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    U = Xd @ A.T
    return X @ W_hat.T + lora_scale(alpha, r) * (U @ B.T), U


def backward_dropout(W_hat, X, A, B, dY, alpha: float, r: int, keep_bits, p: float, round_bf16: bool = True):
    """(dX, dA, dB) in float64 for the layer with dropout on the adapter input."""
    W_hat = np.asarray(W_hat, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    dY = np.asarray(dY, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    s = lora_scale(alpha, r)
    keep = unpack_keep(keep_bits, X.shape[1])
    Xd = dropped_input(X, keep_bits, p, round_bf16)
    G = dY @ B
    U = Xd @ A.T
    dX = dY @ W_hat + np.where(keep, s * (G @ A) * dropout_factor(p), 0.0)
    dA = s * (G.T @ Xd)
    dB = s * (dY.T @ U)
    return dX, dA, dB
