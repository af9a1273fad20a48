"""NF4 blockwise quantization with double-quantized scales -- CPU oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle``): never imported by the product path.

The steps follow the offline base-weight quantization of [QLoRA-入门到精通]
§3(1), in its order, with the level table of §2(3) of the same page and the
quantization section of [X长文] (block scaling, NF4, storage and compute):

1. Level table (``nf4_levels``).  Levels are normal-distribution quantiles:
   the standard normal is cut into slices of equal probability and each slice
   is represented by its median; the grid is dense near 0, sparse in the tails,
   contains an exact 0, has 16 entries and lies in [-1, 1].
   Reading (the pages lose the formula): 16 equal slices of the whole normal
   have medians symmetric about 0 with no zero level, which contradicts "exact
   0".  The plainest construction with every stated property is: cut the lower
   half into 7 equal-probability slices and the upper half into 8, take each
   slice's median, scale each half by its own largest magnitude (so the ends
   are exactly -1 and +1 and the block's absmax element of either sign is
   representable), add the level 0, sort ascending (index 0 = -1, index 15 = +1,
   ascending numbering as in [QLoRA-量化微调] §7.1).  Values are computed in
   float64 (statistics.NormalDist.inv_cdf) and rounded to float32.
2. Blocking: the weight is flattened row-major and cut into blocks of
   ``blocksize`` consecutive values (64 on the hot path; [QLoRA-入门到精通]
   §3(1) names 64 or 256, [X长文] names 64).
3. Scale: s_b = absmax of the block, in float32 (exact).
4. Normalize: x = fl32(w / s_b), IEEE division (so |x| <= 1 exactly).
   Reading for an all-zero block (pages silent): s_b = 0, every x = 0.
5. Nearest level: q = the index of the nearest level to x.  Reading for ties
   (pages silent): the lower index wins.  Decided exactly for every float32 x
   (see ``_nearest_level``).
6. Pack: two 4-bit indices per byte.  Reading for nibble order (pages silent):
   element 2j goes in the high nibble, element 2j+1 in the low nibble, which
   matches reading the printed binary code of the worked example from the left
   ([QLoRA-量化微调] §7.1).  Layout: row-major [d_out][d_in/2].
7. Double quantization: the float32 block scales are gathered and quantized to
   8 bits ([QLoRA-入门到精通] §3(1); [X长文] storage paragraph, about 4.13
   bits per weight).  Readings (pages silent on format): groups of
   ``dq_blocksize`` consecutive scales (256 on the hot path); each group keeps
   one float32 constant c_g = max of its scales (scales are >= 0, so absmax is
   the max); codes are unsigned 8-bit linear on [0, c_g]:
   code = rint_half_even(fl32(fl32(s_b / c_g) * 255)), and 0 when c_g = 0.
   Indices are computed from the exact s_b (step 5 happens before step 7).
8. Dequantize: s'_b = fl32(fl32(code) * fl32(c_g / 255)), then the weight is
   restored as bf16_rne(fl32(T[q] * s'_b)) ([QLoRA-入门到精通] §3(2): table
   value times the block's stored scale, restored to a 16-bit float).  With
   double quantization off (``dq_blocksize == 0``) s'_b = s_b.

Pins (``tests/test_oracle_nf4.py``): the uniform-grid worked example of
[QLoRA-量化微调] §7.1 (0.27 -> index 9 -> 0.304), table invariants and the
median property via an independent CDF (scipy.special.ndtr), exact-rational
brute force of the nearest-level rule around every midpoint, the quantization
error bound, the storage figures (4.5 bits without double quantization,
about 4.13 with it, 48 bits for a group of four), closed-form code values.
"""

from dataclasses import dataclass
from statistics import NormalDist
from typing import Optional

import numpy as np

from .bf16 import round_to_bf16


# ----------------------------------------------------------------------------
# Step 1: level tables
# ----------------------------------------------------------------------------

def nf4_levels() -> np.ndarray:
    """The 16 NF4 levels (float32, ascending, index 7 is exactly 0)."""
    inv = NormalDist().inv_cdf
    neg = [inv((j + 0.5) / 14.0) for j in range(7)]          # 7 slices of the lower half
    pos = [inv(0.5 + (j + 0.5) / 16.0) for j in range(8)]    # 8 slices of the upper half
    neg_scale = max(abs(v) for v in neg)
    pos_scale = max(pos)
    levels = [v / neg_scale for v in neg] + [0.0] + [v / pos_scale for v in pos]
    levels.sort()
    return np.array(levels, dtype=np.float32)


def uniform_levels() -> np.ndarray:
    """16 equally spaced levels on [-1, 1]: -1 + 2i/15 ([QLoRA-量化微调] §7.1)."""
    return np.array([-1.0 + 2.0 * i / 15.0 for i in range(16)], dtype=np.float32)


# ----------------------------------------------------------------------------
# Steps 2-7: quantize
# ----------------------------------------------------------------------------

@dataclass
class Quantized:
    shape: tuple            # (d_out, d_in) of the original weight
    blocksize: int
    dq_blocksize: int       # 0 = double quantization off
    q: np.ndarray           # uint8 [numel]   4-bit indices (unpacked)
    packed: np.ndarray      # uint8 [d_out][d_in/2]  two indices per byte
    scales: np.ndarray      # float32 [nb]    first-level absmax scales s_b
    codes: Optional[np.ndarray]   # uint8 [nb] 8-bit scale codes (None if DQ off)
    consts: Optional[np.ndarray]  # float32 [ng] second-level constants c_g (None if DQ off)


def _nearest_level(x: np.ndarray, levels: np.ndarray, chunk: int = 1 << 20) -> np.ndarray:
    """Index of the nearest level to each x; ties go to the lower index.

    For an ascending table the distance to the levels first falls then rises
    with the index, so the nearest index is the number of adjacent pairs
    (T_k, T_k+1) for which x is strictly closer to T_k+1, i.e. for which
    2x > T_k + T_k+1.  Both sides are exact in float64 (2x is a float32 times
    two; the sum of two float32 levels in [-1, 1] fits in 53 bits), so the
    comparison is exact for every float32 x, including tiny ones.
    """
    lv = levels.astype(np.float64)
    assert np.all(np.diff(lv) > 0), "levels must be strictly ascending"
    pair_sum = lv[:-1] + lv[1:]
    out = np.empty(x.shape, dtype=np.uint8)
    flat_x = x.reshape(-1)
    flat_o = out.reshape(-1)
    for s in range(0, flat_x.size, chunk):
        two_x = 2.0 * flat_x[s:s + chunk].astype(np.float64)
        flat_o[s:s + chunk] = np.sum(two_x[:, None] > pair_sum[None, :], axis=1)
    return out


def _normalize(blocks: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Step 4: x = fl32(w / s_b) for every value of a block, by IEEE float32
    division (the normalized value X_block / scale of [QLoRA-入门到精通]
    §3(1)); rows of ``blocks`` are blocks, ``scales`` their absmax.  A block
    whose scale is 0 (all zero) gives x = 0."""
    safe = np.where(scales > 0, scales, np.float32(1.0)).astype(np.float32)
    x = (blocks / safe[:, None]).astype(np.float32)
    x[scales == 0] = np.float32(0.0)
    return x


def quantize(W, levels: Optional[np.ndarray] = None, blocksize: int = 64,
             dq_blocksize: int = 256) -> Quantized:
    """Blockwise absmax quantization of a float32 weight to 4-bit level indices.

    ``W`` is [d_out][d_in] (or 1-D); ``levels`` defaults to ``nf4_levels()``.
    The flattened size must be a multiple of ``blocksize``.
    """
    if levels is None:
        levels = nf4_levels()
    W = np.asarray(W, dtype=np.float32)
    shape = W.shape if W.ndim == 2 else (1, W.size)
    w = W.reshape(-1)
    assert np.all(np.isfinite(w)), "inputs must be finite"
    assert w.size % blocksize == 0, "numel must be a multiple of the block size"
    assert w.size % 2 == 0

    # step 2: blocks of consecutive values
    blocks = w.reshape(-1, blocksize)
    # step 3: absmax scale per block (float32, exact)
    scales = np.max(np.abs(blocks), axis=1).astype(np.float32)
    # step 4: normalize by IEEE float32 division; all-zero block -> x = 0
    x = _normalize(blocks, scales)
    # step 5: nearest level index
    q = _nearest_level(x, levels).reshape(-1)
    # step 6: two indices per byte, element 2j in the high nibble
    packed = ((q[0::2].astype(np.uint8) << 4) | q[1::2].astype(np.uint8)).astype(np.uint8)
    packed = packed.reshape(shape[0], shape[1] // 2)

    # step 7: double quantization of the scales
    codes = consts = None
    if dq_blocksize:
        nb = scales.size
        ng = -(-nb // dq_blocksize)
        consts = np.zeros(ng, dtype=np.float32)
        codes = np.zeros(nb, dtype=np.uint8)
        for g in range(ng):
            sg = scales[g * dq_blocksize:(g + 1) * dq_blocksize]
            c = np.float32(np.max(sg))
            consts[g] = c
            if c > 0:
                ratio = (sg / c).astype(np.float32)                    # fl32(s_b / c_g)
                scaled = (ratio * np.float32(255.0)).astype(np.float32)  # fl32(ratio * 255)
                codes[g * dq_blocksize:(g + 1) * dq_blocksize] = np.clip(np.rint(scaled), 0, 255)
    return Quantized(shape=tuple(shape), blocksize=blocksize, dq_blocksize=dq_blocksize,
                     q=q, packed=packed, scales=scales, codes=codes, consts=consts)


# ----------------------------------------------------------------------------
# Step 8: dequantize
# ----------------------------------------------------------------------------

def restored_scales(Q: Quantized) -> np.ndarray:
    """s'_b: the scale each block is restored with (float32)."""
    if not Q.dq_blocksize:
        return Q.scales.copy()
    g = np.arange(Q.scales.size) // Q.dq_blocksize
    step = (Q.consts / np.float32(255.0)).astype(np.float32)      # fl32(c_g / 255)
    return (Q.codes.astype(np.float32) * step[g]).astype(np.float32)


def unpack(packed: np.ndarray) -> np.ndarray:
    """uint8 bytes -> 4-bit indices in element order (high nibble first)."""
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    q = np.empty(p.size * 2, dtype=np.uint8)
    q[0::2] = p >> 4
    q[1::2] = p & 0x0F
    return q


def dequantize(Q: Quantized, levels: Optional[np.ndarray] = None, to_bf16: bool = True,
               rows=None, cols=None) -> np.ndarray:
    """Restore the weight: T[q] * s'_b in float32, then rounded to bfloat16.

    Returns float32 [d_out][d_in] (bf16-valued when ``to_bf16``).  Indices are
    read back from the packed bytes, so packing is exercised too.  For a 2-D
    weight whose rows are whole blocks, ``rows`` (or ``cols``) restores only
    those rows [len(rows)][d_in] (or columns [d_out][len(cols)]), each element
    with the same arithmetic as the whole restore.
    """
    if levels is None:
        levels = nf4_levels()
    q = unpack(Q.packed)
    s = restored_scales(Q)
    if rows is None and cols is None:
        vals = levels[q].reshape(-1, Q.blocksize)
        w = (vals * s[:, None]).astype(np.float32)
        shape = Q.shape
    else:
        N, K = Q.shape
        if K % Q.blocksize:
            raise ValueError("a row/column subset needs rows made of whole blocks")
        q2, s2 = q.reshape(N, K), s.reshape(N, K // Q.blocksize)
        if rows is not None:
            r = np.asarray(rows)
            qq, ss = q2[r], s2[r][:, np.arange(K) // Q.blocksize]
        else:
            c = np.asarray(cols)
            qq, ss = q2[:, c], s2[:, c // Q.blocksize]
        w = (levels[qq] * ss).astype(np.float32)
        shape = w.shape
    if to_bf16:
        w = round_to_bf16(w)
    return w.reshape(shape)


# ----------------------------------------------------------------------------
# Storage accounting
# ----------------------------------------------------------------------------

def storage_bits_per_weight(numel: int, blocksize: int = 64, dq_blocksize: int = 256,
                            index_bits: int = 4) -> float:
    """Average stored bits per weight: indices + scale metadata.

    Double quantization off: one float32 scale per block.  On: one 8-bit code
    per block plus one float32 constant per group of ``dq_blocksize`` blocks
    ([X长文] storage paragraph; [QLoRA-量化微调] §7.1 extended calculation).
    """
    nb = -(-numel // blocksize)
    if not dq_blocksize:
        meta = 32 * nb
    else:
        ng = -(-nb // dq_blocksize)
        meta = 8 * nb + 32 * ng
    return (index_bits * numel + meta) / numel
