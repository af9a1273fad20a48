"""Oracle's own bfloat16 rounding (TEST INFRASTRUCTURE ONLY; see ``oracle``).

The compute type of the layer is bfloat16: the base weight is restored to a
16-bit float before it enters the product ([QLoRA-入门到精通] §3(2), on-demand
dequantization to BF16/FP16; [LoRA-QLoRA-工程] §8, compute dtype bfloat16).
bfloat16 is the upper half of an IEEE binary32; rounding is to nearest, ties to
even.  Inputs are finite (NaN handling is out of scope).

Pinned in ``tests/test_oracle_bf16.py`` against torch's own float32->bfloat16
conversion (an independent library routine) and against hand-picked tie cases.
"""

import numpy as np


def round_to_bf16(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 arrays whose low 16 bits are zero.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = (bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    out = (rounded << np.uint64(16)).astype(np.uint32)
    return out.view(np.float32).reshape(f.shape)


def bits_to_float(bits) -> np.ndarray:
    """Interpret uint16 bfloat16 bit patterns as float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def float_to_bits(x) -> np.ndarray:
    """float32 -> uint16 bfloat16 bit patterns, rounding to nearest even."""
    r = round_to_bf16(x)
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
