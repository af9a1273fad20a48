"""Pins for the QLoRA layer oracle (CPU): forward, backward, merge."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import lora, nf4
from oracle.bf16 import bits_to_float
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _restored(W):
    return nf4.dequantize(nf4.quantize(W)).astype(np.float64)


# --------------------------------------------------------------------------
# P2: the sales tables through the layer (exact)
# --------------------------------------------------------------------------

def _sales_layer(cols, rows, alpha=None):
    """W = 0 (quantizes to the zero level), alpha = r so s = 1, X = identity:
    then Y = (B A)^T exactly.  Embedded in a 64 x 64 layer."""
    r = len(cols)
    B = np.zeros((64, r))
    A = np.zeros((r, 64))
    for i, (c, w) in enumerate(zip(cols, rows)):
        B[:len(c), i] = c
        A[i, :len(w)] = w
    W_hat = _restored(np.zeros((64, 64), np.float32))
    assert np.all(W_hat == 0)
    X = np.eye(64)
    Y, U = lora.forward(W_hat, X, A, B, alpha=float(r) if alpha is None else alpha, r=r)
    return Y, B, A


def test_sales_table_rank1_and_rank2():
    g = json.load(open(os.path.join(GOLDEN, "sales_tables.json")))
    c1, r1 = g["rank1"]["column"], g["rank1"]["row"]
    c2, r2 = g["rank2_extra_pattern"]["column"], g["rank2_extra_pattern"]["row"]
    # rank 1: 3 x 4 table = column x row; 12 numbers from 3 + 4 = 7
    Y, B, A = _sales_layer([c1], [r1])
    table = Y.T[:3, :4]
    np.testing.assert_array_equal(table, [[10, 20, 20, 10], [20, 40, 40, 20], [30, 60, 60, 30]])
    assert np.linalg.matrix_rank(table) == g["rank1"]["rank"]
    assert len(c1) + len(r1) == g["rank1"]["numbers_stored"] and table.size == g["rank1"]["numbers_in_table"]
    for i in range(3):                      # each row is the same row vector scaled by the store size
        np.testing.assert_array_equal(table[i], c1[i] * np.array(r1))
    # rank 2: the promotion pattern added
    Y, B, A = _sales_layer([c1, c2], [r1, r2])
    table2 = Y.T[:3, :4]
    np.testing.assert_array_equal(table2, [[10, 20, 25, 15], [20, 40, 40, 20], [30, 60, 70, 40]])
    assert np.linalg.matrix_rank(table2) == g["rank2_extra_pattern"]["rank"]
    sv = np.linalg.svd(table2, compute_uv=False)
    assert sv[1] > 1e-6 * sv[0] and sv[2] < 1e-9 * sv[0]


def test_sales_table_scaled_by_alpha_over_r():
    # alpha = 2r -> the LoRA branch is doubled: Y = 2 (B A)^T exactly
    g = json.load(open(os.path.join(GOLDEN, "sales_tables.json")))
    Y, B, A = _sales_layer([g["rank1"]["column"]], [g["rank1"]["row"]], alpha=2.0)
    np.testing.assert_array_equal(Y.T[:3, :4], 2 * np.array([[10, 20, 20, 10], [20, 40, 40, 20], [30, 60, 60, 30]]))


# --------------------------------------------------------------------------
# P3: B = 0 -> output equals the base model; dA = 0, dB != 0
# --------------------------------------------------------------------------

def test_b_zero_identity():
    inp = workloads.layer_inputs(128, 256, 8, 4, seed=5)
    W_hat = _restored(inp["W"])
    X, A, dY = (bits_to_float(inp[k]) for k in ("X", "A", "dY"))
    B0 = np.zeros((128, 4))
    Y, _ = lora.forward(W_hat, X, A, B0, 8.0, 4)
    Yb, _ = lora.forward(W_hat, X, None, None, 8.0, 0)
    np.testing.assert_array_equal(Y, Yb)
    np.testing.assert_array_equal(Yb, X @ W_hat.T)
    dX, dA, dB = lora.backward(W_hat, X, A, B0, dY, 8.0, 4)
    assert np.all(dA == 0)
    assert np.abs(dB).max() > 0                 # A != 0, so B gets a gradient at step one
    np.testing.assert_array_equal(dX, dY @ W_hat)


# --------------------------------------------------------------------------
# P4: merged weight equals the two-branch result
# --------------------------------------------------------------------------

def test_merge_equivalence():
    inp = workloads.layer_inputs(192, 128, 12, 8, seed=6)
    W_hat = _restored(inp["W"])
    X, A, B = (bits_to_float(inp[k]) for k in ("X", "A", "B"))
    Y, _ = lora.forward(W_hat, X, A, B, 16.0, 8)
    Wm = lora.merged_weight(W_hat, A, B, 16.0, 8)
    np.testing.assert_allclose(X @ Wm.T, Y, rtol=1e-12, atol=1e-12 * np.abs(Y).max())
    # merging happens on the restored 16-bit weight: the 4-bit indices are untouched
    assert not np.array_equal(Wm, W_hat)


def test_scale_is_alpha_over_r():
    assert lora.lora_scale(16.0, 8) == 2.0 and lora.lora_scale(32.0, 16) == 2.0
    assert lora.lora_scale(16.0, 64) == 0.25
    assert lora.lora_scale(1.0, 3) == float(np.float32(1.0) / np.float32(3.0))


# --------------------------------------------------------------------------
# P9: backward = derivative of forward
# --------------------------------------------------------------------------

def _tiny(seed=9):
    rng = np.random.default_rng(seed)
    T, K, N, r = 3, 64, 64, 2
    W_hat = _restored((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    X = rng.standard_normal((T, K))
    A = rng.standard_normal((r, K)) / r
    B = rng.standard_normal((N, r)) * 0.3
    dY = rng.standard_normal((T, N))
    return W_hat, X, A, B, dY, 5.0, r


def test_backward_matches_finite_differences():
    W_hat, X, A, B, dY, alpha, r = _tiny()
    dX, dA, dB = lora.backward(W_hat, X, A, B, dY, alpha, r)

    def loss(X_, A_, B_):
        Y, _ = lora.forward(W_hat, X_, A_, B_, alpha, r)
        return float(np.sum(Y * dY))

    h = 1e-6
    rng = np.random.default_rng(1)
    for name, arr, grad in (("X", X, dX), ("A", A, dA), ("B", B, dB)):
        for _ in range(12):
            idx = tuple(rng.integers(0, n) for n in arr.shape)
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            args_p = {"X": (p, A, B), "A": (X, p, B), "B": (X, A, p)}[name]
            args_m = {"X": (m, A, B), "A": (X, m, B), "B": (X, A, m)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def test_backward_matches_torch_autograd_float64():
    W_hat, X, A, B, dY, alpha, r = _tiny(11)
    s = float(np.float32(alpha) / np.float32(r))          # alpha / r, computed here independently
    tX = torch.tensor(X, requires_grad=True)
    tA = torch.tensor(A, requires_grad=True)
    tB = torch.tensor(B, requires_grad=True)
    tW = torch.tensor(W_hat)                      # frozen: no grad
    Y = torch.nn.functional.linear(tX, tW) + s * torch.nn.functional.linear(torch.nn.functional.linear(tX, tA), tB)
    Y.backward(torch.tensor(dY))
    dX, dA, dB = lora.backward(W_hat, X, A, B, dY, alpha, r)
    np.testing.assert_allclose(dX, tX.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dA, tA.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dB, tB.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert tW.grad is None
    Yo, _ = lora.forward(W_hat, X, A, B, alpha, r)
    np.testing.assert_allclose(Yo, Y.detach().numpy(), rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# P7: trainable parameter count r (d_in + d_out)
# --------------------------------------------------------------------------

def test_trainable_parameter_count():
    d, r = 4096, 8
    A = np.zeros((r, d))
    B = np.zeros((d, r))
    assert A.size + B.size == 65536
    assert round(100 * (A.size + B.size) / (d * d), 2) == 0.39


# --------------------------------------------------------------------------
# LoRA dropout on the adapter input ([LoRA-QLoRA-工程] §4.3)
# --------------------------------------------------------------------------

def _drop_case(p=0.25, seed=21):
    import workloads
    rng = np.random.default_rng(seed)
    T, K, N, r = 5, 16, 12, 3
    W = rng.standard_normal((N, K))
    X = rng.standard_normal((T, K))
    A = rng.standard_normal((r, K))
    B = rng.standard_normal((N, r))
    dY = rng.standard_normal((T, N))
    keep = workloads.dropout_keep_bits(T, K, p, seed)
    return W, X, A, B, dY, keep, r


def test_dropout_keep_bit_order():
    bits = np.array([[0b00000101, 0b10000000]], np.uint8)
    k = lora.unpack_keep(bits, 16)
    assert list(np.flatnonzero(k[0])) == [0, 2, 15]


def test_dropout_p0_all_kept_is_the_plain_layer():
    from oracle.bf16 import round_to_bf16
    W, X, A, B, dY, _, r = _drop_case()
    X = round_to_bf16(X.astype(np.float32)).astype(np.float64)      # exact bf16 inputs
    keep = np.full((X.shape[0], X.shape[1] // 8), 0xFF, np.uint8)
    Y0, U0 = lora.forward(W, X, A, B, 4.0, r)
    Y1, U1 = lora.forward_dropout(W, X, A, B, 4.0, r, keep, 0.0)
    np.testing.assert_array_equal(Y0, Y1)
    np.testing.assert_array_equal(U0, U1)
    for a, b in zip(lora.backward(W, X, A, B, dY, 4.0, r), lora.backward_dropout(W, X, A, B, dY, 4.0, r, keep, 0.0)):
        np.testing.assert_array_equal(a, b)


def test_dropout_all_dropped_leaves_the_base_branch():
    W, X, A, B, dY, _, r = _drop_case()
    keep = np.zeros((X.shape[0], X.shape[1] // 8), np.uint8)
    Y, U = lora.forward_dropout(W, X, A, B, 4.0, r, keep, 0.5)
    assert not U.any()
    np.testing.assert_array_equal(Y, X @ W.T)
    dX, dA, dB = lora.backward_dropout(W, X, A, B, dY, 4.0, r, keep, 0.5)
    np.testing.assert_array_equal(dX, dY @ W)
    assert not dA.any() and not dB.any()


def _autograd_dropout(W, X, A, B, dY, keep_bool, c, s):
    import torch
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    Xt, At, Bt = t(X), t(A), t(B)
    M = torch.tensor(keep_bool, dtype=torch.float64)
    Y = Xt @ torch.tensor(W).T + s * ((Xt * M * c) @ At.T) @ Bt.T
    (Y * torch.tensor(dY)).sum().backward()
    return Xt.grad.numpy(), At.grad.numpy(), Bt.grad.numpy()


def test_dropout_backward_matches_torch_autograd_float64():
    W, X, A, B, dY, keep, r = _drop_case()
    alpha, p = 6.0, 0.25
    want = _autograd_dropout(W, X, A, B, dY, lora.unpack_keep(keep, X.shape[1]), lora.dropout_factor(p),
                             lora.lora_scale(alpha, r))
    got = lora.backward_dropout(W, X, A, B, dY, alpha, r, keep, p, round_bf16=False)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, rtol=1e-12, atol=1e-12)


def test_dropout_planted_mistake_fails_autograd():
    # the adapter's share of dX without the mask (a plausible slip) differs from autograd
    W, X, A, B, dY, keep, r = _drop_case()
    alpha, p = 6.0, 0.25
    want = _autograd_dropout(W, X, A, B, dY, lora.unpack_keep(keep, X.shape[1]), lora.dropout_factor(p),
                             lora.lora_scale(alpha, r))[0]
    s = lora.lora_scale(alpha, r)
    unmasked = dY @ W + s * ((dY @ B) @ A) * lora.dropout_factor(p)
    assert not np.allclose(unmasked, want, rtol=1e-6)


def test_dropped_input_rounding():
    # kept values are bf16(fl32(x * c)), c = fl32(1 / (1 - p)); checked against
    # torch's own float32 product and float32 -> bfloat16 conversion
    import torch
    X = np.array([[1.0, 3.0, -0.7, 2.5, 0.1, 0.2, 0.3, 0.4]])
    keep = np.array([[0b11111011]], np.uint8)
    Xd = lora.dropped_input(X, keep, 0.1)
    c = torch.tensor(1.0, dtype=torch.float32) / (torch.tensor(1.0, dtype=torch.float32) - torch.tensor(0.1, dtype=torch.float32))
    want = (torch.tensor(X[0], dtype=torch.float32) * c).to(torch.bfloat16).to(torch.float64).numpy()
    want[2] = 0.0
    np.testing.assert_array_equal(Xd[0], want)
