"""GPU parity for LoRA dropout on the adapter's input ("LoRA 与 QLoRA：把大模型
微调拆成可负担的工程" §4.3; §8 configuration lora_dropout 0.05): the layer
with a seeded keep mask against the oracle's forward_dropout /
backward_dropout, on every kernel path; p = 0 with every element kept and
every element dropped reduce to the plain layer and to the base branch."""

import numpy as np
import pytest

import workloads
from gpu_helpers import TOL, dev_bf16, dev_f32, host_bf16_to_f64, normwise_err, say
from oracle import lora as olora
from oracle import nf4 as onf4
from oracle.bf16 import bits_to_float

pytestmark = pytest.mark.gpu


def _dev_keep(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits)).cuda()


def _run(inp, r, alpha, keep_bits, p, with_u=True):
    import nf4_bit_quantized_amd as q
    import torch
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]))
    X, A, B, dY = (dev_bf16(inp[k]) for k in ("X", "A", "B", "dY"))
    keep = _dev_keep(keep_bits)
    Y, U = q.qlora_linear_fwd(packed, codes, consts, X, A, B, alpha, keep=keep, p=p)
    dX, dA, dB = q.qlora_linear_bwd(packed, codes, consts, X, A, B, alpha, dY, U_in=U if with_u else None,
                                    keep=keep, p=p)
    torch.cuda.synchronize()
    return {"Y": Y, "U": U, "dX": dX, "dA": dA, "dB": dB}


def _host(g):
    return {"Y": host_bf16_to_f64(g["Y"]), "dX": host_bf16_to_f64(g["dX"]),
            "U": g["U"].cpu().numpy().astype(np.float64), "dA": g["dA"].cpu().numpy().astype(np.float64),
            "dB": g["dB"].cpu().numpy().astype(np.float64)}


DROP_CASES = [
    # (d_out, d_in, T, r, alpha, p, seed)
    (256, 256, 16, 8, 16.0, 0.05, 100),    # the pages' rate; tiled kernels
    (256, 512, 4, 16, 32.0, 0.1, 101),     # few tokens: few-token forward, split-contraction adapters
    (192, 320, 100, 3, 5.0, 0.5, 102),     # odd rank, ragged tokens
    (320, 448, 600, 24, 8.0, 0.05, 103),   # streaming adapter products
    (256, 256, 40, 128, 16.0, 0.3, 104),   # largest rank
]


@pytest.mark.parametrize("d_out,d_in,T,r,alpha,p,seed", DROP_CASES)
def test_dropout_parity(d_out, d_in, T, r, alpha, p, seed):
    say(f"dropout d_out={d_out} d_in={d_in} T={T} r={r} p={p}")
    inp = workloads.layer_inputs(d_out, d_in, T, r, seed)
    keep = workloads.dropout_keep_bits(T, d_in, p, seed)
    W_hat = onf4.dequantize(onf4.quantize(inp["W"]))
    X, A, B, dY = (bits_to_float(inp[k]) for k in ("X", "A", "B", "dY"))
    Y, U = olora.forward_dropout(W_hat, X, A, B, alpha, r, keep, p)
    dX, dA, dB = olora.backward_dropout(W_hat, X, A, B, dY, alpha, r, keep, p)
    want = {"Y": Y, "U": U, "dX": dX, "dA": dA, "dB": dB}
    for with_u in (True, False):
        got = _host(_run(inp, r, alpha, keep, p, with_u))
        errs = {k: normwise_err(got[k], want[k]) for k in want}
        say("  errors", with_u, {k: f"{v:.2e}" for k, v in errs.items()})
        for k, v in errs.items():
            assert v <= TOL, (k, v)


def test_dropout_p0_all_kept_is_the_plain_layer():
    import nf4_bit_quantized_amd as q
    import torch
    from gpu_helpers import gpu_layer
    inp = workloads.layer_inputs(256, 320, 48, 16, seed=105)
    keep = np.full((48, 40), 0xFF, np.uint8)
    g = _run(inp, 16, 16.0, keep, 0.0)
    ref = gpu_layer(inp, 16, 16.0)
    np.testing.assert_array_equal(host_bf16_to_f64(g["Y"]), ref["Y"])
    for k in ("U", "dA", "dB"):
        np.testing.assert_array_equal(g[k].cpu().numpy().astype(np.float64), ref[k])
    # dX: the base share a is rounded to bf16 before the adapter's share b is
    # added, an extra error of up to half a bf16 step of a (2^-9 |a|) on top of
    # the final rounding; where a and b cancel that is large against a + b, so
    # the bound is normwise, with |a| <= |a + b| + |b| and |b| small here
    assert normwise_err(host_bf16_to_f64(g["dX"]), ref["dX"]) <= 2.0 ** -6


def test_dropout_all_dropped_is_the_base_branch():
    import nf4_bit_quantized_amd as q
    import torch
    inp = workloads.layer_inputs(256, 320, 48, 16, seed=106)
    keep = np.zeros((48, 40), np.uint8)
    g = _run(inp, 16, 16.0, keep, 0.5)
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]))
    X, dY = dev_bf16(inp["X"]), dev_bf16(inp["dY"])
    Y0, _ = q.qlora_linear_fwd(packed, codes, consts, X, None, None, 0.0)
    dX0, _, _ = q.qlora_linear_bwd(packed, codes, consts, X, None, None, 0.0, dY)
    torch.cuda.synchronize()
    assert torch.equal(g["Y"].view(torch.int16), Y0.view(torch.int16))
    assert torch.equal(g["dX"].view(torch.int16), dX0.view(torch.int16))
    assert not g["U"].any() and not g["dA"].any() and not g["dB"].any()


def test_dropout_with_accumulation():
    import nf4_bit_quantized_amd as q
    import torch
    inp = workloads.layer_inputs(192, 256, 64, 8, seed=107)
    keep = _dev_keep(workloads.dropout_keep_bits(64, 256, 0.1, 107))
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]))
    X, A, B, dY = (dev_bf16(inp[k]) for k in ("X", "A", "B", "dY"))
    _, U = q.qlora_linear_fwd(packed, codes, consts, X, A, B, 8.0, keep=keep, p=0.1)
    _, dA1, dB1 = q.qlora_linear_bwd(packed, codes, consts, X, A, B, 8.0, dY, U_in=U, keep=keep, p=0.1)
    dA = torch.ones_like(dA1)
    dB = torch.full_like(dB1, -0.5)
    q.qlora_linear_bwd(packed, codes, consts, X, A, B, 8.0, dY, U_in=U, dA=dA, dB=dB, keep=keep, p=0.1,
                       accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(dA, 1.0 + dA1)
    assert torch.equal(dB, -0.5 + dB1)
