"""GPU parity for several layers that share their input
("LoRA 与 QLoRA：把大模型微调拆成可负担的工程" §8: LoRA on every linear module,
so the projections of one input arrive together): each layer's Y and U, dA
and dB, and the summed dX against the oracle.  With at most 16 tokens all
weights stream in one launch; with more, weights that are whole 256-column
tiles and share one table run as ONE forward product over their columns, and
the backward computes dX as ONE product whose contraction runs over every
weight's rows (each layer's rank-r term a tail of the same fp32 sum, rounded
once); other sets run layer by layer."""

import numpy as np
import pytest

import workloads
from gpu_helpers import (TOL, dev_bf16, dev_f32, elementwise_stats, host_bf16_to_f64, normwise_err,
                         oracle_sampled, say)
from oracle import lora as olora
from oracle import nf4 as onf4
from oracle.bf16 import bits_to_float

pytestmark = pytest.mark.gpu


def _layers(shapes, K, T, r, seed, tables=None):
    import nf4_bit_quantized_amd as q
    tables = tables or [0] * len(shapes)
    X = workloads.layer_inputs(64, K, T, 1, seed, with_dy=False)["X"]
    out = []
    for i, N in enumerate(shapes):
        inp = workloads.layer_inputs(N, K, T, r, seed + 1 + i, with_dy=False)
        pk, cd, cs = q.qlora_quantize_nf4(dev_f32(inp["W"]), table=tables[i])
        out.append(dict(inp=inp, dev=(pk, cd, cs, dev_bf16(inp["A"]) if r else None, dev_bf16(inp["B"]) if r else None),
                        levels=None if tables[i] == 0 else onf4.uniform_levels()))
    return X, out


@pytest.mark.parametrize("T", [1, 4, 16])
def test_qkv_shaped_few_tokens_match_oracle(T):
    """Query 512 rows, key and value 128 rows each (grouped-query shapes), K = 512, r = 8."""
    import nf4_bit_quantized_amd as q
    import torch
    K, r, alpha = 512, 8, 16.0
    say(f"multi T={T}")
    Xb, layers = _layers([512, 128, 128], K, T, r, seed=110)
    outs = q.qlora_linear_fwd_multi([l["dev"] for l in layers], dev_bf16(Xb), alpha)
    torch.cuda.synchronize()
    X = bits_to_float(Xb)
    for l, (Y, U) in zip(layers, outs):
        W_hat = onf4.dequantize(onf4.quantize(l["inp"]["W"], levels=l["levels"]), levels=l["levels"])
        Yo, Uo = olora.forward(W_hat, X, bits_to_float(l["inp"]["A"]), bits_to_float(l["inp"]["B"]), alpha, r)
        ey, eu = normwise_err(host_bf16_to_f64(Y), Yo), normwise_err(U.cpu().numpy().astype(np.float64), Uo)
        say(f"  Y {ey:.2e} U {eu:.2e}")
        assert ey <= TOL and eu <= TOL


def test_mixed_tables_and_rank_zero():
    import nf4_bit_quantized_amd as q
    import torch
    K, T = 256, 3
    Xb, layers = _layers([256, 64], K, T, 0, seed=120, tables=[1, 0])
    outs = q.qlora_linear_fwd_multi([l["dev"] for l in layers], dev_bf16(Xb), 0.0, tables=[1, 0])
    torch.cuda.synchronize()
    X = bits_to_float(Xb)
    for l, (Y, U) in zip(layers, outs):
        assert U is None
        W_hat = onf4.dequantize(onf4.quantize(l["inp"]["W"], levels=l["levels"]), levels=l["levels"])
        assert normwise_err(host_bf16_to_f64(Y), X @ W_hat.T) <= TOL


def test_many_tokens_run_layer_by_layer_bit_identical():
    import nf4_bit_quantized_amd as q
    import torch
    K, T, r, alpha = 320, 40, 16, 8.0
    Xb, layers = _layers([192, 64, 64], K, T, r, seed=130)
    X = dev_bf16(Xb)
    outs = q.qlora_linear_fwd_multi([l["dev"] for l in layers], X, alpha)
    sep = [q.qlora_linear_fwd(*l["dev"][:3], X, l["dev"][3], l["dev"][4], alpha) for l in layers]
    torch.cuda.synchronize()
    for (Y, U), (Ys, Us) in zip(outs, sep):
        assert torch.equal(Y.view(torch.int16), Ys.view(torch.int16))
        assert torch.equal(U, Us)


def test_gqa_70b_shapes_one_token():
    """Query 8192x8192 with key and value 1024x8192 at one token, r = 64,
    against separate calls (the same kernels, within the bar)."""
    import nf4_bit_quantized_amd as q
    import torch
    K, T, r, alpha = 8192, 1, 64, 16.0
    g = torch.Generator(device="cuda").manual_seed(140)
    layers = []
    for N in (8192, 1024, 1024):
        pk, cd, cs = q.qlora_quantize_nf4(torch.randn(N, K, device="cuda", generator=g) * 0.02)
        A = (torch.randn(r, K, device="cuda", generator=g) / r).to(torch.bfloat16)
        B = (torch.randn(N, r, device="cuda", generator=g) * 0.01).to(torch.bfloat16)
        layers.append((pk, cd, cs, A, B))
    X = torch.randn(T, K, device="cuda", generator=g).to(torch.bfloat16)
    outs = q.qlora_linear_fwd_multi(layers, X, alpha)
    sep = [q.qlora_linear_fwd(*l[:3], X, l[3], l[4], alpha) for l in layers]
    torch.cuda.synchronize()
    for (Y, U), (Ys, Us) in zip(outs, sep):
        e = normwise_err(Y.float().cpu().numpy().astype(np.float64), Ys.float().cpu().numpy().astype(np.float64))
        say(f"  Y vs separate {e:.2e}")
        assert e <= TOL
        assert torch.equal(U, Us)


@pytest.mark.parametrize("T", [16, 40])
def test_caller_buffers_match_allocated_outputs(T):
    """Outputs and workspace given by the caller (filled with 0xFF bytes
    first) hold what the allocating call returns, bit for bit: the one-launch
    path at 16 tokens, layer by layer at 40."""
    import nf4_bit_quantized_amd as q
    import torch
    K, r, alpha = 512, 8, 16.0
    say(f"multi caller buffers T={T}")
    Xb, layers = _layers([512, 128, 128], K, T, r, seed=150)
    devs = [l["dev"] for l in layers]
    X = dev_bf16(Xb)
    ref = q.qlora_linear_fwd_multi(devs, X, alpha)
    bufs = [(torch.full((T, N), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16),
             torch.full((T, r), -1, dtype=torch.int32, device="cuda").view(torch.float32)) for N in (512, 128, 128)]
    import ctypes
    n_b = ctypes.c_size_t()
    descs = (q.Nf4Desc * 3)(*[q._stored_desc(*d[:3], 0) for d in devs])
    q._check(q.lib().qlora_multi_fwd_workspace_bytes(3, descs, T, r, ctypes.byref(n_b)), "ws")
    ws = torch.full((max(1, n_b.value),), 0xFF, dtype=torch.uint8, device="cuda")
    got = q.qlora_linear_fwd_multi(devs, X, alpha, workspace=ws, outs=bufs)
    torch.cuda.synchronize()
    for (Yr, Ur), (Yg, Ug), (Yb, Ub) in zip(ref, got, bufs):
        assert Yg.data_ptr() == Yb.data_ptr() and Ug.data_ptr() == Ub.data_ptr()
        assert torch.equal(Yr.view(torch.int16), Yg.view(torch.int16))
        assert torch.equal(Ur.view(torch.int32), Ug.view(torch.int32))


@pytest.mark.parametrize("T", [4, 40, 600])
def test_backward_of_layers_sharing_x(T):
    """dX is the sum of the layers' shares; dA, dB are each layer's own."""
    import nf4_bit_quantized_amd as q
    import torch
    K, r, alpha = 320, 8, 16.0
    say(f"multi backward T={T}")
    Xb, layers = _layers([192, 64, 64], K, T, r, seed=150)
    X = dev_bf16(Xb)
    dYs_b = [workloads.layer_inputs(l["dev"][0].shape[0], K, T, 1, 160 + i)["dY"] for i, l in enumerate(layers)]
    dYs = [dev_bf16(b) for b in dYs_b]
    outs = q.qlora_linear_fwd_multi([l["dev"] for l in layers], X, alpha)
    dX, grads = q.qlora_linear_bwd_multi([l["dev"] for l in layers], X, alpha, dYs, U_ins=[o[1] for o in outs])
    torch.cuda.synchronize()
    Xf = bits_to_float(Xb)
    want_dx = 0.0
    for l, dyb, (dA, dB) in zip(layers, dYs_b, grads):
        W_hat = onf4.dequantize(onf4.quantize(l["inp"]["W"]))
        dXo, dAo, dBo = olora.backward(W_hat, Xf, bits_to_float(l["inp"]["A"]), bits_to_float(l["inp"]["B"]),
                                       bits_to_float(dyb), alpha, r)
        want_dx = want_dx + dXo
        ea = normwise_err(dA.cpu().numpy().astype(np.float64), dAo)
        eb = normwise_err(dB.cpu().numpy().astype(np.float64), dBo)
        assert ea <= TOL and eb <= TOL, (ea, eb)
    ex = normwise_err(host_bf16_to_f64(dX), want_dx)
    say(f"  dX {ex:.2e}")
    assert ex <= TOL


@pytest.mark.parametrize("T", [4, 40])
def test_backward_caller_buffers_match_allocated_outputs(T):
    """dX, dA and dB given by the caller (filled with 0xFF bytes first) are
    overwritten with what the allocating call returns, bit for bit."""
    import nf4_bit_quantized_amd as q
    import torch
    K, r, alpha = 320, 8, 16.0
    say(f"multi backward caller buffers T={T}")
    Xb, layers = _layers([192, 64, 64], K, T, r, seed=170)
    X = dev_bf16(Xb)
    devs = [l["dev"] for l in layers]
    dYs = [dev_bf16(workloads.layer_inputs(d[0].shape[0], K, T, 1, 180 + i)["dY"]) for i, d in enumerate(devs)]
    Us = [o[1] for o in q.qlora_linear_fwd_multi(devs, X, alpha)]
    dX_ref, g_ref = q.qlora_linear_bwd_multi(devs, X, alpha, dYs, U_ins=Us)
    dX = torch.full((T, K), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    grads = [(torch.full((r, K), -1, dtype=torch.int32, device="cuda").view(torch.float32),
              torch.full((d[0].shape[0], r), -1, dtype=torch.int32, device="cuda").view(torch.float32)) for d in devs]
    dX_got, g_got = q.qlora_linear_bwd_multi(devs, X, alpha, dYs, U_ins=Us, dX=dX, grads=grads)
    torch.cuda.synchronize()
    assert dX_got.data_ptr() == dX.data_ptr()
    assert torch.equal(dX_ref.view(torch.int16), dX.view(torch.int16))
    for (dAr, dBr), (dAg, dBg), (dAb, dBb) in zip(g_ref, g_got, grads):
        assert dAg.data_ptr() == dAb.data_ptr() and dBg.data_ptr() == dBb.data_ptr()
        assert torch.equal(dAr.view(torch.int32), dAg.view(torch.int32))
        assert torch.equal(dBr.view(torch.int32), dBg.view(torch.int32))


def _launches(kernel):
    """Launch counts of ``kernel`` recorded since the last read (trace stays on)."""
    import nf4_bit_quantized_amd as q
    return q.qlora_trace_read(reset=True).get(kernel, (0, 0.0))[0]


def _traced(kernels):
    import nf4_bit_quantized_amd as q
    q.qlora_trace_select(kernels)
    q.qlora_trace_read(reset=True)


def _untrace():
    import nf4_bit_quantized_amd as q
    q.qlora_trace_enable(False)
    q.qlora_trace_read(reset=True)


# every weight whole 256-column tiles, at least one round of them (256) in all: the one-product forward
FUSED_FWD = [
    # (T, r, tables, shapes)
    (8192, 16, (0, 0, 0), (2048, 1024, 1024)),       # 32 x 16 tiles
    (8229, 12, (0, 0, 0), (2048, 1024, 1024)),       # ragged last tile row, rank not a multiple of 8
    (8229, 16, (1, 1, 1), (1024, 2048, 1024)),       # the uniform table for all three
    (8192, 8, (0, 0), (2048, 2048)),                 # two weights
    (8192, 16, (0, 0, 0, 0), (2048, 1024, 512, 512)),  # four weights
]


@pytest.mark.parametrize("T,r,tables,shapes", FUSED_FWD)
def test_one_forward_product_over_whole_tile_weights(T, r, tables, shapes):
    """K = 128 (two contraction steps plus the tails): Y and U of every layer
    against the oracle, normwise and elementwise; the forward product runs
    as one launch."""
    import nf4_bit_quantized_amd as q
    import torch
    K, alpha = 128, 16.0
    say(f"fused multi fwd T={T} r={r} tables={tables} shapes={shapes}")
    Xb, layers = _layers(list(shapes), K, T, r, seed=200 + T % 97 + r, tables=list(tables))
    _traced(["fwd_gemm"])
    try:
        outs = q.qlora_linear_fwd_multi([l["dev"] for l in layers], dev_bf16(Xb), alpha, tables=list(tables))
        torch.cuda.synchronize()
        assert _launches("fwd_gemm") == 1
    finally:
        _untrace()
    X = bits_to_float(Xb)
    for l, (Y, U) in zip(layers, outs):
        W_hat = onf4.dequantize(onf4.quantize(l["inp"]["W"], levels=l["levels"]), levels=l["levels"])
        Yo, Uo = olora.forward(W_hat, X, bits_to_float(l["inp"]["A"]), bits_to_float(l["inp"]["B"]), alpha, r)
        Yg = host_bf16_to_f64(Y)
        ey, eu = normwise_err(Yg, Yo), normwise_err(U.cpu().numpy().astype(np.float64), Uo)
        st = elementwise_stats(Yg, Yo)
        say(f"  Y {ey:.2e} {st} U {eu:.2e}")
        assert ey <= TOL and eu <= 1e-5
        assert st["share_above_1e-2"] < 1e-3


@pytest.mark.parametrize("shapes,tables", [((2048, 1024, 960), (0, 0, 0)),   # one weight not whole tiles
                                           ((2048, 1024, 1024), (0, 1, 0)),  # two tables
                                           ((1024, 1024, 1024, 1024), (0, 0, 0, 0))])  # too few tiles at T = 2048
def test_forward_runs_per_weight_otherwise(shapes, tables):
    """Sets the one-product forward does not take: one launch per weight,
    each layer's Y against the oracle."""
    import nf4_bit_quantized_amd as q
    import torch
    K, r, alpha = 128, 16, 16.0
    T = 2048 if len(shapes) == 4 else 8192
    say(f"multi fwd per weight shapes={shapes} tables={tables}")
    Xb, layers = _layers(list(shapes), K, T, r, seed=230 + len(shapes), tables=list(tables))
    _traced(["fwd_gemm"])
    try:
        outs = q.qlora_linear_fwd_multi([l["dev"] for l in layers], dev_bf16(Xb), alpha, tables=list(tables))
        torch.cuda.synchronize()
        assert _launches("fwd_gemm") == len(shapes)
    finally:
        _untrace()
    X = bits_to_float(Xb)
    for l, (Y, U) in zip(layers, outs):
        W_hat = onf4.dequantize(onf4.quantize(l["inp"]["W"], levels=l["levels"]), levels=l["levels"])
        Yo, _ = olora.forward(W_hat, X, bits_to_float(l["inp"]["A"]), bits_to_float(l["inp"]["B"]), alpha, r)
        assert normwise_err(host_bf16_to_f64(Y), Yo) <= TOL


@pytest.mark.parametrize("T,r,tables,shapes", [(300, 8, (0, 0, 0), (256, 128, 64)),
                                               (1000, 12, (1, 1), (192, 320)),
                                               (1000, 12, (1, 0), (192, 320)),
                                               (300, 0, (0, 0, 0, 0), (64, 128, 64, 192)),
                                               (300, 8, (0, 1, 0), (256, 128, 64))])
def test_backward_dx_over_weights(T, r, tables, shapes):
    """dX summed over the layers against the oracle's sum (normwise, and per
    element within the bf16 rounding bound of the path), dA and dB per layer;
    one dX product when the tables agree, one per layer (each adding to dX)
    when they do not."""
    import nf4_bit_quantized_amd as q
    import torch
    K, alpha = 384, 16.0
    say(f"multi bwd T={T} r={r} tables={tables} shapes={shapes}")
    Xb, layers = _layers(list(shapes), K, T, r, seed=260 + T % 89 + r, tables=list(tables))
    X = dev_bf16(Xb)
    dYs_b = [workloads.layer_inputs(N, K, T, 1, 290 + i)["dY"] for i, N in enumerate(shapes)]
    devs = [l["dev"] for l in layers]
    outs = q.qlora_linear_fwd_multi(devs, X, alpha, tables=list(tables))
    _traced(["dx_gemm"])
    try:
        dX, grads = q.qlora_linear_bwd_multi(devs, X, alpha, [dev_bf16(b) for b in dYs_b],
                                             U_ins=[o[1] for o in outs] if r else None, tables=list(tables))
        torch.cuda.synchronize()
        assert _launches("dx_gemm") == (1 if len(set(tables)) == 1 else len(shapes))
    finally:
        _untrace()
    Xf = bits_to_float(Xb)
    want_dx, absum = 0.0, 0.0
    for l, dyb, (dA, dB) in zip(layers, dYs_b, grads):
        W_hat = onf4.dequantize(onf4.quantize(l["inp"]["W"], levels=l["levels"]), levels=l["levels"])
        dXo, dAo, dBo = olora.backward(W_hat, Xf, bits_to_float(l["inp"]["A"]) if r else None,
                                       bits_to_float(l["inp"]["B"]) if r else None, bits_to_float(dyb), alpha, r)
        want_dx, absum = want_dx + dXo, absum + np.abs(dXo)
        if r:
            ea = normwise_err(dA.cpu().numpy().astype(np.float64), dAo)
            eb = normwise_err(dB.cpu().numpy().astype(np.float64), dBo)
            assert ea <= TOL and eb <= TOL, (ea, eb)
    got = host_bf16_to_f64(dX)
    ex, st = normwise_err(got, want_dx), elementwise_stats(got, want_dx)
    # rounding bound per element: one product rounds dX to bf16 once; layer
    # by layer, each product's share is rounded to bf16 and, from the second
    # layer on, added to dX and rounded again (2n - 1 roundings).  Each is
    # within 2^-8 (bf16's unit roundoff) of a value no larger than the sum of the layers' |shares|;
    # fp32 accumulation adds far less
    nround = 1 if len(set(tables)) == 1 else 2 * len(shapes) - 1
    bound = nround * 2.0 ** -8 * absum * 1.01 + 1e-4 * np.max(np.abs(want_dx))
    worst = float(np.max(np.abs(got - want_dx) / bound))
    say(f"  dX {ex:.2e} {st} rounding-bound ratio {worst:.3f}")
    assert ex <= TOL
    assert worst <= 1.0
    if len(set(tables)) == 1:
        assert st["share_above_1e-2"] < 1e-2


@pytest.mark.timeout(600)
@pytest.mark.parametrize("group", ["qkv", "gate_up"])
def test_stack_projection_groups_full_size_sampled(group):
    """The 65B-class layer's projection groups at 4096 tokens, r = 64,
    alpha = 16: query/key/value (three 8192 x 8192 weights) and gate/up (two
    22016 x 8192), each group through one forward product and one dX
    product.  Sampled against the oracle: Y and dB on 16 output rows of
    every layer, dX (summed over the group) and dA on 32 input columns."""
    import nf4_bit_quantized_amd as q
    import torch
    shapes = {"qkv": (8192, 8192, 8192), "gate_up": (22016, 22016)}[group]
    K, T, r, alpha = 8192, 4096, 64, 16.0
    say(f"stack group {group}: drawing inputs")
    inps = [workloads.layer_inputs(N, K, T, r, seed=400 + i) for i, N in enumerate(shapes)]
    Xb = inps[0]["X"]
    devs = []
    for inp in inps:
        pk, cd, cs = q.qlora_quantize_nf4(dev_f32(inp["W"]))
        devs.append((pk, cd, cs, dev_bf16(inp["A"]), dev_bf16(inp["B"])))
    X = dev_bf16(Xb)
    dYs = [dev_bf16(inp["dY"]) for inp in inps]
    _traced(["fwd_gemm", "dx_gemm"])
    try:
        outs = q.qlora_linear_fwd_multi(devs, X, alpha)
        dX, grads = q.qlora_linear_bwd_multi(devs, X, alpha, dYs, U_ins=[o[1] for o in outs])
        torch.cuda.synchronize()
        st = q.qlora_trace_read(reset=True)
        assert st["fwd_gemm"][0] == 1 and st["dx_gemm"][0] == 1, st
    finally:
        _untrace()
    say("  gpu done; oracle on sampled outputs")
    rng = np.random.default_rng(17 + len(shapes))
    cols = np.sort(rng.choice(K, size=32, replace=False))
    ci = torch.as_tensor(cols, device="cuda")
    Xf = bits_to_float(Xb)
    want_dx, errs = 0.0, []
    for i, (inp, (Y, _), (dA, dB)) in enumerate(zip(inps, outs, grads)):
        rows = np.sort(rng.choice(shapes[i], size=16, replace=False))
        ri = torch.as_tensor(rows, device="cuda")
        Q = onf4.quantize(inp["W"])
        A, B, dY = (bits_to_float(inp[k]) for k in ("A", "B", "dY"))
        want = oracle_sampled(Q, Xf, A, B, dY, alpha, r, rows, cols)
        want_dx = want_dx + want["dX"]
        got = {"Y": host_bf16_to_f64(Y.index_select(1, ri)),
               "dB": dB.index_select(0, ri).cpu().numpy().astype(np.float64),
               "dA": dA.index_select(1, ci).cpu().numpy().astype(np.float64)}
        for k in got:
            e = normwise_err(got[k], want[k])
            errs.append((i, k, e))
            say(f"  layer {i} {k} {e:.2e}")
    ex = normwise_err(host_bf16_to_f64(dX.index_select(1, ci)), want_dx)
    say(f"  dX {ex:.2e}")
    assert ex <= TOL
    for i, k, e in errs:
        assert e <= TOL, (i, k, e)
