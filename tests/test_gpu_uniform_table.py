"""GPU parity for the uniform 16-level table (-1 + 2i/15 on [-1, 1], the grid
of the worked example in "7、QLoRA 量化微调" §7.1) through the same kernels as
the NF4 table: quantization bit-exact, the worked example's printed values,
forward/backward within the bar, and both exports."""

import numpy as np
import pytest

import workloads
from gpu_helpers import (TOL, assert_quant_bit_exact, dev_bf16, dev_f32, gpu_layer, host_bf16_to_f64,
                         normwise_err, oracle_layer, say, sweep_blocks)
from oracle import nf4 as onf4
from oracle.bf16 import bits_to_float, float_to_bits

pytestmark = pytest.mark.gpu

UNIFORM = 1


def _quant_host(packed, codes, consts):
    return {"packed_h": packed.cpu().numpy(), "codes_h": codes.cpu().numpy(), "consts_h": consts.cpu().numpy()}


@pytest.mark.parametrize("d_out,d_in", [(256, 256), (64, 320), (1024, 1024)])
def test_uniform_quantize_bit_exact(d_out, d_in):
    import nf4_bit_quantized_amd as q
    import torch
    say(f"uniform quantize {d_out}x{d_in}")
    inp = workloads.layer_inputs(d_out, d_in, 1, 1, seed=40, with_dy=False)
    Q = onf4.quantize(inp["W"], levels=onf4.uniform_levels())
    g = q.qlora_quantize_nf4(dev_f32(inp["W"]), table=UNIFORM)
    torch.cuda.synchronize()
    assert_quant_bit_exact(_quant_host(*g), Q)


@pytest.mark.parametrize("scales", [(1.0,), (0.0123, 7.25, 1.0e-3), (1.0e-39, 3.0e30)])
def test_uniform_threshold_sweep_bit_exact(scales):
    """Every decision point of the uniform table (midpoints of adjacent
    levels, zero among them) and 40 float32 neighbours on each side."""
    import nf4_bit_quantized_amd as q
    import torch
    _, thr = q.qlora_table_levels(UNIFORM)
    W = np.concatenate([sweep_blocks(sc, thr) for sc in scales])
    pad = (-W.size) % (64 * 64)
    W = np.concatenate([W, np.zeros(pad, np.float32)]).reshape(64, -1)
    say(f"uniform threshold sweep {scales} W {W.shape}")
    Q = onf4.quantize(W, levels=onf4.uniform_levels())
    g = q.qlora_quantize_nf4(dev_f32(W), table=UNIFORM)
    torch.cuda.synchronize()
    assert_quant_bit_exact(_quant_host(*g), Q)


def test_uniform_worked_example_on_gpu():
    """The group [0.27, 0.58, -0.75, 1.52] at the head of a 64-weight block
    (the rest zero): 0.27 takes index 9 (binary 1001, level 0.2) and restores
    to 0.2 * 1.52 = 0.304 up to the bf16 rounding; the other three take 10, 4
    and 15, packed element 0 in the high nibble."""
    import nf4_bit_quantized_amd as q
    import torch
    W = np.zeros((64, 64), np.float32)
    W[0, :4] = [0.27, 0.58, -0.75, 1.52]
    Q = onf4.quantize(W, levels=onf4.uniform_levels())
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(W), table=UNIFORM)
    W_hat = q.qlora_dequantize_nf4(packed, codes, consts, table=UNIFORM)
    torch.cuda.synchronize()
    assert_quant_bit_exact(_quant_host(packed, codes, consts), Q)
    p = packed.cpu().numpy().reshape(-1)
    assert p[0] >> 4 == 9 and list(p[:2]) == [0x9A, 0x4F]
    got = W_hat.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, float_to_bits(onf4.dequantize(Q, levels=onf4.uniform_levels())))
    w0 = float(bits_to_float(got[0, :1])[0])
    assert abs(w0 - 0.304) <= 2.0 ** -9                     # one bf16 step in [0.25, 0.5)


UNIFORM_CASES = [
    # (d_out, d_in, T, r, alpha, seed): few-token path, fused GEMMs, streaming adapter products
    (256, 256, 1, 8, 16.0, 41),
    (128, 448, 4, 8, 16.0, 42),
    (256, 256, 16, 8, 16.0, 43),
    (192, 320, 100, 3, 5.0, 44),
    (256, 192, 600, 24, 8.0, 45),
    (4160, 256, 2, 16, 16.0, 46),
]


@pytest.mark.parametrize("d_out,d_in,T,r,alpha,seed", UNIFORM_CASES)
def test_uniform_fwd_bwd_parity(d_out, d_in, T, r, alpha, seed):
    say(f"uniform fwd/bwd d_out={d_out} d_in={d_in} T={T} r={r} seed={seed}")
    inp = workloads.layer_inputs(d_out, d_in, T, r, seed)
    o = oracle_layer(inp, r, alpha, levels=onf4.uniform_levels())
    g = gpu_layer(inp, r, alpha, table=UNIFORM)
    assert_quant_bit_exact(g, o["Q"])
    errs = {k: normwise_err(g[k], o[k]) for k in ("Y", "U", "dX", "dA", "dB")}
    say("  errors", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= TOL, (k, v)
    # the table is really in use: the NF4 table gives another restored weight
    n = gpu_layer(inp, r, alpha, do_bwd=False)
    assert not np.array_equal(n["packed_h"], g["packed_h"])


def test_uniform_exports():
    import nf4_bit_quantized_amd as q
    import torch
    from oracle import lora as olora
    d_out, d_in, r, alpha = 256, 4160, 16, 16.0
    say(f"uniform exports {d_out}x{d_in} r={r}")
    inp = workloads.layer_inputs(d_out, d_in, 1, r, seed=47)
    lv = onf4.uniform_levels()
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]), table=UNIFORM)
    Wh = q.qlora_dequantize_nf4(packed, codes, consts, table=UNIFORM)
    Wm = q.qlora_merge_lora(packed, codes, consts, dev_bf16(inp["A"]), dev_bf16(inp["B"]), alpha, table=UNIFORM)
    torch.cuda.synchronize()
    W_hat = onf4.dequantize(onf4.quantize(inp["W"], levels=lv), levels=lv)
    np.testing.assert_array_equal(Wh.view(torch.int16).cpu().numpy().view(np.uint16), float_to_bits(W_hat))
    want = olora.merged_weight(W_hat, bits_to_float(inp["A"]), bits_to_float(inp["B"]), alpha, r)
    got = host_bf16_to_f64(Wm)
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 7)
    tol = step + 2.0 ** -20 * (np.abs(W_hat) + np.abs(want - W_hat))
    worst = float(np.max(np.abs(got - want) / tol))
    say(f"  worst error {worst:.3f} of the bound")
    assert worst <= 1.0
