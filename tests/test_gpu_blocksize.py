"""GPU parity for absmax blocks of 128 and 256 weights ("QLoRA技术从入门到精通"
§3(1): the weight is cut into blocks of e.g. 64 or 256 values, each with its
own scale), through the same kernels as blocks of 64: quantization bit-exact
(blocks that span two rows and ragged last groups included), forward and
backward on every kernel path, and both exports."""

import numpy as np
import pytest

import workloads
from gpu_helpers import (TOL, assert_quant_bit_exact, dev_bf16, dev_f32, gpu_layer, host_bf16_to_f64,
                         normwise_err, oracle_layer, say, sweep_blocks)
from oracle import nf4 as onf4
from oracle.bf16 import bits_to_float, float_to_bits

pytestmark = pytest.mark.gpu


def _host(packed, codes, consts):
    return {"packed_h": packed.cpu().numpy(), "codes_h": codes.cpu().numpy(), "consts_h": consts.cpu().numpy()}


@pytest.mark.parametrize("bs", [128, 256])
@pytest.mark.parametrize("d_out,d_in", [(256, 256), (64, 320), (192, 1024), (4096, 4096)])
def test_quantize_bit_exact(bs, d_out, d_in):
    import nf4_bit_quantized_amd as q
    import torch
    say(f"quantize bs={bs} {d_out}x{d_in}")
    W = workloads.layer_inputs(d_out, d_in, 1, 1, seed=70, with_dy=False)["W"]
    g = q.qlora_quantize_nf4(dev_f32(W), blocksize=bs)
    torch.cuda.synchronize()
    assert g[1].numel() == d_out * d_in // bs
    assert_quant_bit_exact(_host(*g), onf4.quantize(W, blocksize=bs))


@pytest.mark.parametrize("bs", [128, 256])
def test_quantize_16bit_weight_and_uniform_table(bs):
    import nf4_bit_quantized_amd as q
    import torch
    W = workloads.layer_inputs(192, 320, 1, 1, seed=71, with_dy=False)["W"]
    bits = workloads.bf16_bits(W)
    Wd = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    a = q.qlora_quantize_nf4(Wd, blocksize=bs)
    b = q.qlora_quantize_nf4(dev_f32(W), blocksize=bs, table=1)
    torch.cuda.synchronize()
    assert_quant_bit_exact(_host(*a), onf4.quantize(bits_to_float(bits).astype(np.float32), blocksize=bs))
    assert_quant_bit_exact(_host(*b), onf4.quantize(W, blocksize=bs, levels=onf4.uniform_levels()))


@pytest.mark.parametrize("bs", [128, 256])
def test_quantize_threshold_sweep_bit_exact(bs):
    """Every decision threshold and its float32 neighbours inside blocks of bs
    weights whose absmax is exactly a chosen scale, at several scales."""
    import nf4_bit_quantized_amd as q
    import torch
    _, thr = q.qlora_nf4_levels()
    W = np.concatenate([sweep_blocks(sc, thr, per=bs - 1, bs=bs) for sc in (1.0, 0.0123, 7.25, 1.0e-39, 3.0e30)])
    pad = (-W.size) % (64 * 64)
    W = np.concatenate([W, np.zeros(pad, np.float32)]).reshape(64, -1)
    say(f"sweep bs={bs} W {W.shape}")
    g = q.qlora_quantize_nf4(dev_f32(W), blocksize=bs)
    torch.cuda.synchronize()
    assert_quant_bit_exact(_host(*g), onf4.quantize(W, blocksize=bs))


BS_CASES = [
    # (d_out, d_in, T, r, alpha, seed, bs)
    (256, 512, 4, 8, 16.0, 72, 128),      # few-token kernel
    (256, 512, 4, 8, 16.0, 73, 256),
    (192, 1024, 16, 64, 16.0, 74, 128),   # few-token kernel, four token rows per load
    (4160, 256, 2, 16, 16.0, 75, 256),    # few-token kernel, two 16-row tiles per workgroup
    (256, 8192, 9, 16, 16.0, 80, 128),    # few-token kernel, contraction split over two workgroups
    (128, 320, 3, 8, 16.0, 76, 128),      # rows not whole blocks: tiled kernel for few tokens
    (256, 256, 100, 16, 32.0, 77, 256),   # tiled kernels
    (192, 320, 150, 64, 16.0, 78, 128),   # tiled kernels, blocks spanning rows
    (320, 448, 600, 24, 8.0, 79, 256),    # streaming adapter products
]


@pytest.mark.parametrize("d_out,d_in,T,r,alpha,seed,bs", BS_CASES)
def test_fwd_bwd_parity(d_out, d_in, T, r, alpha, seed, bs):
    say(f"fwd/bwd bs={bs} d_out={d_out} d_in={d_in} T={T} r={r}")
    inp = workloads.layer_inputs(d_out, d_in, T, r, seed)
    o = oracle_layer(inp, r, alpha, Q=onf4.quantize(inp["W"], blocksize=bs))
    g = gpu_layer(inp, r, alpha, blocksize=bs)
    assert_quant_bit_exact(g, o["Q"])
    errs = {k: normwise_err(g[k], o[k]) for k in ("Y", "U", "dX", "dA", "dB")}
    say("  errors", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= TOL, (k, v)


@pytest.mark.parametrize("bs", [128, 256])
@pytest.mark.parametrize("d_out,d_in", [(192, 320), (256, 4160)])
def test_exports(bs, d_out, d_in):
    import nf4_bit_quantized_amd as q
    import torch
    from oracle import lora as olora
    r, alpha = 16, 16.0
    say(f"exports bs={bs} {d_out}x{d_in}")
    inp = workloads.layer_inputs(d_out, d_in, 1, r, seed=80)
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]), blocksize=bs)
    Wh = q.qlora_dequantize_nf4(packed, codes, consts)
    Wm = q.qlora_merge_lora(packed, codes, consts, dev_bf16(inp["A"]), dev_bf16(inp["B"]), alpha)
    torch.cuda.synchronize()
    W_hat = onf4.dequantize(onf4.quantize(inp["W"], blocksize=bs))
    np.testing.assert_array_equal(Wh.view(torch.int16).cpu().numpy().view(np.uint16), float_to_bits(W_hat))
    want = olora.merged_weight(W_hat, bits_to_float(inp["A"]), bits_to_float(inp["B"]), alpha, r)
    got = host_bf16_to_f64(Wm)
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 7)
    tol = step + 2.0 ** -20 * (np.abs(W_hat) + np.abs(want - W_hat))
    worst = float(np.max(np.abs(got - want) / tol))
    say(f"  worst error {worst:.3f} of the bound")
    assert worst <= 1.0
