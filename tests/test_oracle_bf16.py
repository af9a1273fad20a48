"""Pin the oracle's bfloat16 rounding against torch's conversion (CPU)."""

import numpy as np
import torch

from oracle.bf16 import round_to_bf16, float_to_bits, bits_to_float


def _torch_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_random_values_match_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * s for s in (1e-3, 0.02, 1.0, 300.0)])
    np.testing.assert_array_equal(float_to_bits(x), _torch_bits(x))


def test_ties_round_to_even():
    # 1 + 2^-8 is exactly halfway between bf16 1.0 and 1 + 2^-7: ties to even -> 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6 -> 1 + 2^-6 (even mantissa)
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -20], np.float32)
    r = round_to_bf16(x)
    assert r[0] == 1.0 and r[1] == 1 + 2 ** -6 and r[2] == -1.0 and r[3] == 1 + 2 ** -7
    np.testing.assert_array_equal(float_to_bits(x), _torch_bits(x))


def test_bits_roundtrip():
    b = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        f = bits_to_float(b)
    finite = np.isfinite(f)
    np.testing.assert_array_equal(float_to_bits(f[finite].astype(np.float32)), b[finite])
