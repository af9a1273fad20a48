"""Pins for the NF4 quantization oracle (CPU only).

Each test checks ``oracle.nf4`` against something other than itself: a value
printed on the pages (tests/golden/), a closed form, an independent library
routine, or exact-rational brute force.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import ndtr  # independent normal CDF (Cephes), not statistics.NormalDist

from oracle import nf4
from oracle.bf16 import round_to_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# P1: the uniform-grid worked example (printed values)
# --------------------------------------------------------------------------

def test_uniform_worked_example_printed_values():
    g = _golden("uniform_worked_example.json")
    p = g["printed"]
    lv = nf4.uniform_levels()
    assert lv.size == p["levels_count"]
    assert abs(float(lv[9]) - 0.2) < 1e-7                      # -1 + 9*2/15
    Q = nf4.quantize(np.array(g["group"], np.float32), levels=lv, blocksize=4, dq_blocksize=0)
    assert Q.scales[0] == np.float32(p["scale"])               # absmax of the group
    x0 = np.float32(g["group"][0]) / Q.scales[0]
    assert round(float(x0), 4) == p["first_normalized"]         # 0.27 / 1.52 ~ 0.1776
    assert int(Q.q[0]) == p["first_index"]
    assert format(int(Q.q[0]), "04b") == p["first_index_binary"]
    assert abs(float(lv[Q.q[0]]) - p["first_level"]) < 1e-7
    w = nf4.dequantize(Q, levels=lv, to_bf16=False).reshape(-1)
    assert abs(float(w[0]) - p["first_restored"]) < 1e-6       # 0.2 * 1.52
    assert round(abs(float(w[0]) - 0.27), 3) == p["first_abs_error"]


def test_uniform_worked_example_whole_group_by_hand():
    # Derived by hand from the page's rule (not printed on the page):
    # 0.58/1.52 = 0.3816 -> nearest of {0.3333 (i=10), 0.4667 (i=11)} is i=10
    # -0.75/1.52 = -0.4934 -> nearest of {-0.6 (i=3), -0.4667 (i=4)} is i=4
    # 1.52/1.52 = 1 -> i=15.  Packed, element 0 in the high nibble: 0x9A, 0x4F.
    lv = nf4.uniform_levels()
    Q = nf4.quantize(np.array([0.27, 0.58, -0.75, 1.52], np.float32), levels=lv, blocksize=4, dq_blocksize=0)
    assert list(Q.q) == [9, 10, 4, 15]
    assert list(Q.packed.reshape(-1)) == [0x9A, 0x4F]
    w = nf4.dequantize(Q, levels=lv, to_bf16=False).reshape(-1)
    np.testing.assert_allclose(w, [0.2 * 1.52, (1 / 3) * 1.52, (-7 / 15) * 1.52, 1.52], rtol=1e-6)


# --------------------------------------------------------------------------
# P6: NF4 table invariants and the median construction
# --------------------------------------------------------------------------

def test_nf4_table_invariants():
    T = nf4.nf4_levels()
    assert T.dtype == np.float32 and T.size == 16
    assert np.all(np.diff(T) > 0)                          # strictly ascending
    assert T[0] == np.float32(-1.0) and T[15] == np.float32(1.0)
    assert np.count_nonzero(T == 0) == 1 and T[7] == 0     # exactly one zero, at index 7
    assert np.sum(T < 0) == 7 and np.sum(T > 0) == 8
    neg_gaps = -np.diff(T[:8][::-1])                        # gaps moving outward from 0, lower side
    pos_gaps = np.diff(T[7:])                               # gaps moving outward from 0, upper side
    assert np.all(np.diff(neg_gaps) > 0), "denser near 0 on the negative side"
    assert np.all(np.diff(pos_gaps) > 0), "denser near 0 on the positive side"


def test_nf4_levels_are_slice_medians_by_independent_cdf():
    """Each level, scaled back by its half's normalizer, sits at the median of
    an equal-probability slice: Phi(level * c) = (j + 1/2)/14 (lower half, 7
    slices) or 1/2 + (j + 1/2)/16 (upper half, 8 slices).  The normalizer is
    recovered from the end level, and Phi is scipy's ndtr (not the inverse
    used to build the table)."""
    T = nf4.nf4_levels().astype(np.float64)
    # normalizer: the outermost slice median, found by bisection on ndtr
    def ppf(p):
        lo, hi = -10.0, 10.0
        for _ in range(200):
            mid = 0.5 * (lo + hi)
            if ndtr(mid) < p:
                lo = mid
            else:
                hi = mid
        return 0.5 * (lo + hi)
    c_neg = -ppf(0.5 / 14)
    c_pos = ppf(0.5 + 7.5 / 16)
    for j in range(7):
        assert abs(ndtr(T[j] * c_neg) - (j + 0.5) / 14) < 1e-7
    for j in range(8):
        assert abs(ndtr(T[8 + j] * c_pos) - (0.5 + (j + 0.5) / 16)) < 1e-7
    # equal probability per slice: 7 slices share the lower half, 8 the upper
    assert abs(7 * (1 / 14) - 0.5) < 1e-15 and abs(8 * (1 / 16) - 0.5) < 1e-15


# --------------------------------------------------------------------------
# Step 5: nearest level, ties to the lower index, by exact rationals
# --------------------------------------------------------------------------

def _nearest_exact(x: float, T) -> int:
    fx = Fraction(float(x))
    best, bd = None, None
    for i, t in enumerate(T):
        d = abs(fx - Fraction(float(t)))
        if bd is None or d < bd:
            best, bd = i, d
    return best


@pytest.mark.parametrize("table", ["nf4", "uniform"])
def test_nearest_level_brute_force_around_every_midpoint(table):
    T = nf4.nf4_levels() if table == "nf4" else nf4.uniform_levels()
    xs = []
    for k in range(15):
        c = np.float32((np.float64(T[k]) + np.float64(T[k + 1])) / 2)
        xs.append(c)
        for direction in (np.float32(np.inf), np.float32(-np.inf)):
            c2 = c
            for _ in range(64):
                c2 = np.nextafter(c2, direction, dtype=np.float32)
                xs.append(c2)
    xs.extend(T.tolist())
    xs.extend([np.float32(-1.0), np.float32(1.0), np.float32(0.0), np.float32(-0.0)])
    xs = np.array(xs, dtype=np.float32)
    got = nf4._nearest_level(xs, T)
    want = np.array([_nearest_exact(x, T) for x in xs])
    np.testing.assert_array_equal(got, want)


def test_nearest_level_random_exact():
    T = nf4.nf4_levels()
    rng = np.random.default_rng(7)
    xs = rng.uniform(-1, 1, 4000).astype(np.float32)
    got = nf4._nearest_level(xs, T)
    want = np.array([_nearest_exact(x, T) for x in xs])
    np.testing.assert_array_equal(got, want)


def test_exact_tie_goes_to_lower_index():
    # x = 0.25 is exactly halfway between the levels 0 and 0.5
    T = np.concatenate([[0.0, 0.5], np.linspace(0.75, 1.0, 14)]).astype(np.float32)
    q = nf4._nearest_level(np.array([0.25], np.float32), T)
    assert q[0] == 0


# --------------------------------------------------------------------------
# Step 4: normalize, x = fl32(w / s), pinned by exact rationals
# --------------------------------------------------------------------------

def _fl32_rne(q: Fraction) -> Fraction:
    """The float32 nearest to the rational q, ties to even (IEEE 754
    round-to-nearest-even written out: 24-bit significands, exponents down to
    -126, then the fixed subnormal spacing 2^-149)."""
    if q == 0:
        return Fraction(0)
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    ulp = Fraction(2) ** (max(e, -126) - 23)
    m = a / ulp
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return (n * ulp) if q > 0 else -(n * ulp)


# fp32 block scales: ordinary, between powers of two, tiny normal, subnormal, huge
NORMALIZE_SCALES = (1.52, 0.0371, 7.77e-6, 123.456, 2.3e-38, 1.0e-40, 3.0e38)


def normalize_walk_blocks(T):
    """Blocks of 64 whose first value is the absmax s and whose other values
    walk +-64 float32 steps across each threshold of T times s."""
    rows, scales = [], []
    for s in NORMALIZE_SCALES:
        s32 = np.float32(s)
        vals = []
        for k in range(15):
            mid = (Fraction(float(T[k])) + Fraction(float(T[k + 1]))) / 2
            c = np.float32(float(_fl32_rne(mid * Fraction(float(s32)))))
            lo = hi = c
            vals.append(c)
            for _ in range(64):
                lo = np.nextafter(lo, np.float32(-np.inf), dtype=np.float32)
                hi = np.nextafter(hi, np.float32(np.inf), dtype=np.float32)
                vals.extend([lo, hi])
        vals = [v for v in vals if abs(float(v)) <= float(s32)]
        for i in range(0, len(vals), 63):
            chunk = vals[i:i + 63]
            chunk = chunk + [np.float32(0.0)] * (63 - len(chunk))
            rows.append([s32] + chunk)
            scales.append(s32)
    return np.array(rows, dtype=np.float32), np.array(scales, dtype=np.float32)


@pytest.mark.parametrize("table", ["nf4", "uniform"])
def test_normalize_is_the_exact_ieee_quotient_at_many_scales(table):
    """[QLoRA-入门到精通] §3(1) normalizes a block as X_block / scale.  For
    block scales that are not powers of two (and for tiny, subnormal and huge
    ones), values within 64 float32 steps of every threshold times s are
    quantized; each index must be the nearest level (ties to the lower index)
    of the correctly rounded quotient, formed here from the exact rational
    w / s.  A reciprocal-multiply normalize, w * fl32(1 / s), moves some of
    these values across a threshold."""
    T = nf4.nf4_levels() if table == "nf4" else nf4.uniform_levels()
    W, scales = normalize_walk_blocks(T)
    Q = nf4.quantize(W, levels=T, blocksize=64, dq_blocksize=0)
    assert np.array_equal(Q.scales, scales)
    got = Q.q.reshape(W.shape)
    Tq = [Fraction(float(t)) for t in T]
    for b in range(W.shape[0]):
        s = Fraction(float(scales[b]))
        for e in range(64):
            x = _fl32_rne(Fraction(float(W[b, e])) / s)
            want = min(range(16), key=lambda i: (abs(x - Tq[i]), i))
            assert got[b, e] == want, (table, float(scales[b]), float(W[b, e]), int(got[b, e]), want)


# --------------------------------------------------------------------------
# Whole quantizer: blocking, scales, packing, zero blocks
# --------------------------------------------------------------------------

def test_block_scales_are_absmax_and_absmax_element_is_exact():
    rng = np.random.default_rng(1)
    W = (rng.standard_normal((8, 128)) * 0.02).astype(np.float32)
    Q = nf4.quantize(W, dq_blocksize=0)
    blocks = W.reshape(-1, 64)
    np.testing.assert_array_equal(Q.scales, np.abs(blocks).max(axis=1))
    Wd = nf4.dequantize(Q, to_bf16=False).reshape(-1, 64)
    amax = np.argmax(np.abs(blocks), axis=1)
    for b in range(blocks.shape[0]):
        assert Wd[b, amax[b]] == blocks[b, amax[b]]       # x = +-1 -> level +-1 -> exact


def test_quantization_error_bound_dq_off():
    # P8: |w - T[q] s| <= (largest half-gap) * s per block (no double quant)
    T = nf4.nf4_levels().astype(np.float64)
    half_gap = np.max(np.diff(T)) / 2
    rng = np.random.default_rng(2)
    W = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    Q = nf4.quantize(W, dq_blocksize=0)
    Wd = nf4.dequantize(Q, to_bf16=False).reshape(-1, 64).astype(np.float64)
    err = np.abs(W.reshape(-1, 64) - Wd)
    bound = half_gap * Q.scales.astype(np.float64)[:, None] * (1 + 1e-6)
    assert np.all(err <= bound)


def test_packing_order_high_nibble_first():
    # hand-built block with known indices: x = T[i] exactly for i = 0..15 (scale 1)
    T = nf4.nf4_levels()
    W = np.concatenate([T, T[::-1], T, T[::-1]]).astype(np.float32).reshape(1, 64)
    Q = nf4.quantize(W, dq_blocksize=0)
    want_q = list(range(16)) + list(range(15, -1, -1)) + list(range(16)) + list(range(15, -1, -1))
    assert list(Q.q) == want_q
    assert Q.packed[0, 0] == 0x01 and Q.packed[0, 1] == 0x23 and Q.packed[0, 8] == 0xFE
    assert list(nf4.unpack(Q.packed)) == want_q


def test_zero_block():
    W = np.zeros((2, 64), np.float32)
    W[1, 5] = 0.5
    Q = nf4.quantize(W, dq_blocksize=256)
    assert np.all(Q.q[:64] == 7)                           # the zero level
    assert Q.scales[0] == 0 and Q.codes[0] == 0
    assert Q.codes[1] == 255 and Q.consts[0] == np.float32(0.5)
    assert np.all(nf4.dequantize(Q)[0] == 0)


def test_all_zero_group_gives_zero_constant_and_codes():
    Q = nf4.quantize(np.zeros((4, 64), np.float32))
    assert Q.consts[0] == 0 and np.all(Q.codes == 0) and np.all(Q.q == 7)


# --------------------------------------------------------------------------
# Step 7: double quantization, closed forms
# --------------------------------------------------------------------------

def test_double_quant_codes_closed_form():
    # Scales constructed directly: block b of row 0 has absmax s_b (one +s_b entry)
    c = np.float32(0.25)
    svals = np.array([c, c / 2, c / 4, 0, c * np.float32(3 / 255), c * np.float32(127.5 / 255)], np.float32)
    W = np.zeros((1, 64 * svals.size), np.float32)
    for b, s in enumerate(svals):
        W[0, 64 * b] = s
    Q = nf4.quantize(W, dq_blocksize=256)
    np.testing.assert_array_equal(Q.scales, svals)
    assert Q.consts[0] == c
    # 255, 127.5 -> 128 (half to even), 63.75 -> 64, 0, 3, 127.5ish -> rint
    exp = [255, 128, 64, 0, 3]
    assert list(Q.codes[:5]) == exp
    r = np.float32(svals[5] / c) * np.float32(255)
    assert Q.codes[5] == int(np.rint(r))


def test_double_quant_restored_scale_within_half_step():
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((32, 1024)) * 0.02).astype(np.float32)
    Q = nf4.quantize(W)                                      # nb = 512 -> 2 groups
    assert Q.consts.size == 2
    s2 = nf4.restored_scales(Q).astype(np.float64)
    g = np.arange(Q.scales.size) // 256
    step = Q.consts.astype(np.float64)[g] / 255
    assert np.all(np.abs(s2 - Q.scales) <= step * 0.5 * (1 + 1e-5))
    for k in range(2):                                       # the group's max scale is restored exactly
        sg = Q.scales[k * 256:(k + 1) * 256]
        assert Q.consts[k] == sg.max()


def test_partial_last_group():
    W = np.ones((1, 64 * 300), np.float32)
    Q = nf4.quantize(W)
    assert Q.consts.size == 2 and Q.codes.size == 300 and np.all(Q.codes == 255)


# --------------------------------------------------------------------------
# Step 8: dequant rounds to bf16 after the float32 product
# --------------------------------------------------------------------------

def test_dequant_is_bf16_of_float32_product():
    rng = np.random.default_rng(4)
    W = (rng.standard_normal((4, 128)) * 0.02).astype(np.float32)
    Q = nf4.quantize(W)
    T = nf4.nf4_levels()
    s2 = nf4.restored_scales(Q)
    q = Q.q.reshape(-1, 64)
    manual = np.empty_like(W.reshape(-1, 64))
    for b in range(q.shape[0]):
        for e in range(64):
            prod = np.float32(T[q[b, e]] * s2[b])
            manual[b, e] = round_to_bf16(np.array([prod], np.float32))[0]
    np.testing.assert_array_equal(nf4.dequantize(Q).reshape(-1, 64), manual)


def test_dequant_row_and_column_subsets_are_elementwise():
    """A subset restore is the whole restore's rows or columns, bit for bit
    (the manual loop above pins the whole restore itself), for NF4 and the
    uniform table, with and without double quantization."""
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((24, 320)) * 0.03).astype(np.float32)
    rows, cols = [0, 5, 23, 7], [0, 63, 64, 319, 128, 200]
    for lv, dq in ((None, 256), (nf4.uniform_levels(), 256), (None, 0)):
        Q = nf4.quantize(W, levels=lv, dq_blocksize=dq)
        full = nf4.dequantize(Q, levels=lv)
        np.testing.assert_array_equal(nf4.dequantize(Q, levels=lv, rows=rows), full[rows])
        np.testing.assert_array_equal(nf4.dequantize(Q, levels=lv, cols=cols), full[:, cols])
        np.testing.assert_array_equal(nf4.dequantize(Q, levels=lv, rows=rows, to_bf16=False),
                                      nf4.dequantize(Q, levels=lv, to_bf16=False)[rows])
    with pytest.raises(ValueError):
        nf4.dequantize(nf4.quantize(np.ones((2, 96), np.float32)), rows=[0])


# --------------------------------------------------------------------------
# P5: storage figures
# --------------------------------------------------------------------------

def test_storage_figures():
    g = _golden("storage_figures.json")
    # group of four with an FP32 scale, no double quant
    assert 4 * 4 + 32 == g["group_of_four_bits_quantized"] and 4 * 16 == g["group_of_four_bits_fp16"]
    assert nf4.storage_bits_per_weight(4, blocksize=4, dq_blocksize=0) * 4 == g["group_of_four_bits_quantized"]
    assert nf4.storage_bits_per_weight(4096 * 4096, 64, 0) == g["block64_no_dq_bits_per_weight"]
    b = nf4.storage_bits_per_weight(4096 * 4096, 64, 256)
    assert round(b, 2) == g["block64_dq_bits_per_weight_approx"]      # 4.127 -> 4.13
    assert abs(16 / b - g["quarter_of_bf16"]) < 0.2                    # about a quarter of bf16
    # the buffers the quantizer returns have exactly these sizes
    W = np.zeros((256, 256), np.float32)
    Q = nf4.quantize(W)
    bits = Q.packed.nbytes * 8 + Q.codes.nbytes * 8 + Q.consts.nbytes * 8
    assert bits == 4 * W.size + 8 * (W.size // 64) + 32 * Q.consts.size


def test_low_rank_count():
    g = _golden("storage_figures.json")["low_rank"]
    d, r = g["d"], g["r"]
    assert d * d == g["full"] and 2 * d * r == g["lowrank"]
    assert round(100 * 2 * d * r / (d * d), 1) == g["percent_approx"]


# --------------------------------------------------------------------------
# Block size ([QLoRA-入门到精通] §3(1): blocks of e.g. 64 or 256 values)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("bs", [128, 256])
def test_larger_blocks_equal_64_when_subblocks_share_the_absmax(bs):
    """If every 64-value piece of a bs-block has the same absmax, the bs-block
    scale equals each piece's and every index is the same as with blocks of 64."""
    rng = np.random.default_rng(7)
    W = np.clip(rng.standard_normal((64, 512)), -3.9, 3.9).astype(np.float32)   # below the planted absmax
    blocks = W.reshape(-1, bs)
    M = np.float32(4.0)
    blocks[:, ::64] = np.where(rng.random((blocks.shape[0], bs // 64)) < 0.5, M, -M)   # absmax M in each piece
    W = blocks.reshape(64, 512)
    Qb = nf4.quantize(W, blocksize=bs)
    Q64 = nf4.quantize(W, blocksize=64)
    np.testing.assert_array_equal(Qb.q, Q64.q)
    np.testing.assert_array_equal(Qb.scales, np.full(W.size // bs, M, np.float32))
    np.testing.assert_array_equal(Q64.scales, np.full(W.size // 64, M, np.float32))


def test_block_128_nearest_level_brute_force():
    rng = np.random.default_rng(8)
    W = (rng.standard_normal((8, 256)) * np.exp(rng.uniform(-3, 3, (8, 1)))).astype(np.float32)
    Q = nf4.quantize(W, blocksize=128)
    T = nf4.nf4_levels().astype(np.float64)
    x = (W.reshape(-1, 128) / Q.scales[:, None]).astype(np.float32).astype(np.float64).reshape(-1)
    d = np.abs(x[:, None] - T[None, :])
    best = np.argmin(d, axis=1)      # argmin takes the lower index on ties, as the layer does
    np.testing.assert_array_equal(Q.q, best)
