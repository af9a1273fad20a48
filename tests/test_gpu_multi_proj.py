"""GPU parity for the forward of several layers that share their input
("LoRA 与 QLoRA：把大模型微调拆成可负担的工程" §8: LoRA on every linear module,
so the projections of one input arrive together): each layer's Y and U
against the oracle; with at most 16 tokens all weights stream in one launch,
otherwise the layers run one after another and match separate calls bit for
bit."""

import numpy as np
import pytest

import workloads
from gpu_helpers import TOL, dev_bf16, dev_f32, host_bf16_to_f64, normwise_err, say
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
