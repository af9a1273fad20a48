"""Planted mistakes in the oracle (CPU only): each plausible slip -- a swapped
nibble order, a tie broken the other way, a dropped scale, a wrong sign, a
transposed operand, floor instead of round -- must make at least one pin fail.
The mistakes are planted in the oracle by monkeypatching, never in GPU code."""

import numpy as np
import pytest

from oracle import lora, nf4
import test_oracle_lora as pins_lora
import test_oracle_nf4 as pins_nf4


def _fails(pin, *args):
    with pytest.raises(AssertionError):
        pin(*args)


def test_pins_pass_unmutated():
    pins_nf4.test_uniform_worked_example_whole_group_by_hand()
    pins_lora.test_backward_matches_finite_differences()


def test_swapped_nibble_order_is_caught(monkeypatch):
    orig = nf4.quantize

    def bad(*a, **k):
        Q = orig(*a, **k)
        p = Q.packed
        Q.packed = ((p & 0x0F) << 4 | (p >> 4)).astype(np.uint8)
        return Q
    monkeypatch.setattr(nf4, "quantize", bad)
    _fails(pins_nf4.test_uniform_worked_example_whole_group_by_hand)


def test_ties_to_upper_index_is_caught(monkeypatch):
    def bad(x, levels, chunk=1 << 20):
        lv = levels.astype(np.float64)
        s = lv[:-1] + lv[1:]
        return np.sum(2.0 * x.reshape(-1, 1).astype(np.float64) >= s[None, :], axis=1).astype(np.uint8).reshape(x.shape)
    monkeypatch.setattr(nf4, "_nearest_level", bad)
    _fails(pins_nf4.test_exact_tie_goes_to_lower_index)


def test_symmetric_sixteen_slice_table_is_caught(monkeypatch):
    from statistics import NormalDist

    def bad():
        v = [NormalDist().inv_cdf((j + 0.5) / 16) for j in range(16)]
        m = max(abs(t) for t in v)
        return np.array([t / m for t in v], np.float32)
    monkeypatch.setattr(nf4, "nf4_levels", bad)
    _fails(pins_nf4.test_nf4_table_invariants)


def test_floor_instead_of_rint_in_scale_codes_is_caught(monkeypatch):
    monkeypatch.setattr(nf4.np, "rint", np.floor)
    _fails(pins_nf4.test_double_quant_codes_closed_form)


def test_missing_bf16_rounding_in_dequant_is_caught(monkeypatch):
    monkeypatch.setattr(nf4, "round_to_bf16", lambda w: w)
    _fails(pins_nf4.test_dequant_is_bf16_of_float32_product)


def test_dropped_lora_scale_is_caught(monkeypatch):
    monkeypatch.setattr(lora, "lora_scale", lambda alpha, r: 1.0)
    _fails(pins_lora.test_backward_matches_torch_autograd_float64)
    _fails(pins_lora.test_sales_table_scaled_by_alpha_over_r)


def test_wrong_sign_in_dx_is_caught(monkeypatch):
    orig = lora.backward

    def bad(W_hat, X, A, B, dY, alpha, r):
        dX, dA, dB = orig(W_hat, X, A, B, dY, alpha, r)
        s = lora.lora_scale(alpha, r)
        return dX - 2 * s * ((dY @ B) @ A), dA, dB
    monkeypatch.setattr(lora, "backward", bad)
    _fails(pins_lora.test_backward_matches_finite_differences)


def test_transposed_operand_in_db_is_caught(monkeypatch):
    orig = lora.backward

    def bad(W_hat, X, A, B, dY, alpha, r):
        dX, dA, dB = orig(W_hat, X, A, B, dY, alpha, r)
        s = lora.lora_scale(alpha, r)
        G = dY @ B                               # uses G where U = X A^T belongs
        return dX, dA, s * (dY.T @ G[:, :r])
    monkeypatch.setattr(lora, "backward", bad)
    _fails(pins_lora.test_backward_matches_finite_differences)


def test_dropped_lora_branch_in_forward_is_caught(monkeypatch):
    monkeypatch.setattr(lora, "forward", lambda W_hat, X, A, B, alpha, r: (np.asarray(X) @ np.asarray(W_hat).T, None))
    _fails(pins_lora.test_sales_table_rank1_and_rank2)


def test_reciprocal_multiply_normalize_is_caught(monkeypatch):
    def bad(blocks, scales):
        safe = np.where(scales > 0, scales, np.float32(1.0)).astype(np.float32)
        inv = (np.float32(1.0) / safe).astype(np.float32)
        x = (blocks * inv[:, None]).astype(np.float32)
        x[scales == 0] = np.float32(0.0)
        return x
    monkeypatch.setattr(nf4, "_normalize", bad)
    with np.errstate(all="ignore"):
        _fails(pins_nf4.test_normalize_is_the_exact_ieee_quotient_at_many_scales, "nf4")
        _fails(pins_nf4.test_normalize_is_the_exact_ieee_quotient_at_many_scales, "uniform")
        # caught by rounding alone: ordinary scales, where 1/s stays finite
        for s in (1.52, 0.0371, 123.456):
            monkeypatch.setattr(pins_nf4, "NORMALIZE_SCALES", (s,))
            _fails(pins_nf4.test_normalize_is_the_exact_ieee_quotient_at_many_scales, "nf4")
