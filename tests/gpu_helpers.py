"""Shared helpers for the GPU parity tests: move seeded inputs to the device,
run the oracle on the same inputs, compare."""

import sys

import numpy as np

from oracle import lora as olora
from oracle import nf4 as onf4
from oracle.bf16 import bits_to_float

# Bar for floating-point outputs: max |gpu - oracle| / max |oracle| per tensor
# (bf16 products, fp32 accumulation; the stated bar is a max relative error of 2e-2).
TOL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev_f32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host_bf16_to_f64(t):
    import torch
    return t.detach().float().cpu().numpy().astype(np.float64)


def normwise_err(got, want) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    scale = np.max(np.abs(want))
    if scale == 0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - want)) / scale)


def elementwise_stats(got, want, floor: float = 1e-3) -> dict:
    """Element-by-element error beside the normwise bar: the largest
    |got - want| / (|want| + floor * max|want|) and the share of elements
    above 1e-2 on that scale (a local fault -- one wrong block scale, a wrong
    tail column -- shows here even when it is small against the tensor's
    largest entry)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.abs(want) + floor * max(float(np.max(np.abs(want))), 1e-300)
    rel = np.abs(got - want) / den
    return {"max_rel": float(np.max(rel)), "share_above_1e-2": float(np.mean(rel > 1e-2))}


def rounding_bound_ratio(got, want, mag, c: float) -> float:
    """Largest |got - want| / (2^-8 |want| + c * mag) over the elements: mag is
    the oracle's result on absolute values (a bound on the sum of the terms'
    magnitudes).  2^-8 |want| covers the output's own bf16 rounding; c * mag
    covers accumulation and the bf16 steps inside the kernel.  At or below 1
    means every element is within that bound; a local fault (one wrong block
    scale, a wrong tail column) exceeds it."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = 2.0 ** -8 * np.abs(want) + c * np.asarray(mag, np.float64) + 1e-30
    return float(np.max(np.abs(got - want) / den))


def oracle_magnitudes(inp, r, alpha, Q=None, levels=None, do_bwd=True):
    """oracle_layer on absolute values: |X| |W_hat|^T + s (|X| |A|^T) |B|^T and
    the backward's counterparts, bounds on each output's sum of term
    magnitudes."""
    if Q is None:
        Q = onf4.quantize(inp["W"], levels=levels)
    W = np.abs(onf4.dequantize(Q, levels=levels).astype(np.float64))
    X = np.abs(bits_to_float(inp["X"]))
    A = np.abs(bits_to_float(inp["A"])) if r > 0 else None
    B = np.abs(bits_to_float(inp["B"])) if r > 0 else None
    Y, U = olora.forward(W, X, A, B, alpha, r)
    out = {"Y": Y, "U": U}
    if do_bwd:
        dX, dA, dB = olora.backward(W, X, A, B, np.abs(bits_to_float(inp["dY"])), alpha, r)
        out.update(dX=dX, dA=dA, dB=dB)
    return out


def oracle_sampled(Q, X, A, B, dY, alpha, r, rows, cols):
    """The oracle's layer on sampled outputs of a full-size weight: Y and dB
    on output rows ``rows``, dX (this layer's share) and dA on input columns
    ``cols``.  olora.forward/backward run on the restored rows (or columns)
    with the operands those outputs depend on, so every value is the
    oracle's own.  X, A, B, dY: float arrays of the exact bf16 values."""
    W_rows = onf4.dequantize(Q, rows=rows).astype(np.float64)   # [rows][K]
    W_cols = onf4.dequantize(Q, cols=cols).astype(np.float64)   # [N][cols]
    Y, _ = olora.forward(W_rows, X, A, B[rows], alpha, r)             # Y[:, rows]
    _, _, dB = olora.backward(W_rows, X, A, B[rows], dY[:, rows], alpha, r)  # dB[rows]
    dX, dA, _ = olora.backward(W_cols, X[:, cols], A[:, cols], B, dY, alpha, r)  # dX[:, cols], dA[:, cols]
    return {"Y": Y, "dB": dB, "dX": dX, "dA": dA}


def oracle_quantized(W):
    return onf4.quantize(W)


def oracle_layer(inp, r, alpha, Q=None, do_bwd=True, levels=None):
    """Oracle forward (+backward) on a workloads.layer_inputs dict (levels:
    None for the NF4 table, else the table's 16 levels)."""
    if Q is None:
        Q = onf4.quantize(inp["W"], levels=levels)
    W_hat = onf4.dequantize(Q, levels=levels).astype(np.float64)
    X = bits_to_float(inp["X"])
    A = bits_to_float(inp["A"]) if r > 0 else None
    B = bits_to_float(inp["B"]) if r > 0 else None
    Y, U = olora.forward(W_hat, X, A, B, alpha, r)
    out = {"Q": Q, "Y": Y, "U": U}
    if do_bwd:
        dY = bits_to_float(inp["dY"])
        dX, dA, dB = olora.backward(W_hat, X, A, B, dY, alpha, r)
        out.update(dX=dX, dA=dA, dB=dB)
    return out


def gpu_layer(inp, r, alpha, do_bwd=True, pass_u=True, table=0, blocksize=64):
    """Quantize + forward (+ backward) through the C ABI; returns host arrays."""
    import torch
    import nf4_bit_quantized_amd as q
    W = dev_f32(inp["W"])
    packed, codes, consts = q.qlora_quantize_nf4(W, table=table, blocksize=blocksize)
    X = dev_bf16(inp["X"])
    A = dev_bf16(inp["A"]) if r > 0 else None
    B = dev_bf16(inp["B"]) if r > 0 else None
    Y, U = q.qlora_linear_fwd(packed, codes, consts, X, A, B, alpha, table=table)
    out = {"packed": packed, "codes": codes, "consts": consts}
    if do_bwd:
        dY = dev_bf16(inp["dY"])
        dX, dA, dB = q.qlora_linear_bwd(packed, codes, consts, X, A, B, alpha, dY,
                                        U_in=U if pass_u else None, table=table)
    torch.cuda.synchronize()
    out["Y"] = host_bf16_to_f64(Y)
    out["U"] = U.cpu().numpy().astype(np.float64) if U is not None else None
    out["packed_h"] = packed.cpu().numpy()
    out["codes_h"] = codes.cpu().numpy()
    out["consts_h"] = consts.cpu().numpy()
    if do_bwd:
        out["dX"] = host_bf16_to_f64(dX)
        out["dA"] = dA.cpu().numpy().astype(np.float64) if dA is not None else None
        out["dB"] = dB.cpu().numpy().astype(np.float64) if dB is not None else None
    return out


def assert_quant_bit_exact(g, Q):
    np.testing.assert_array_equal(g["packed_h"], Q.packed)
    np.testing.assert_array_equal(g["codes_h"], Q.codes)
    np.testing.assert_array_equal(g["consts_h"].view(np.uint32), Q.consts.view(np.uint32))


def sweep_blocks(scale, thr, per=63, width=40, bs=64):
    """Blocks whose absmax is exactly +-scale, holding the float32 neighbours of
    thr[k] * scale for every threshold k (so that fl32(w / scale) walks across
    each decision point)."""
    scale = np.float32(scale)
    vals = []
    for k in range(15):
        c = np.float32(np.float64(thr[k]) * np.float64(scale))
        vals.append(c)
        for d in (np.float32(np.inf), np.float32(-np.inf)):
            v = c
            for _ in range(width):
                v = np.nextafter(v, d, dtype=np.float32)
                vals.append(v)
    vals = np.array(vals, np.float32)
    vals = vals[np.abs(vals) <= scale]
    nblk = -(-vals.size // per)
    W = np.zeros((nblk, bs), np.float32)
    for b in range(nblk):
        chunk = vals[b * per:(b + 1) * per]
        W[b, 0] = scale if b % 2 == 0 else -scale
        W[b, 1:1 + chunk.size] = chunk
    return W.reshape(-1)
