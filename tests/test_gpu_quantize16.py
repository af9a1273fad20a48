"""GPU parity for quantizing a base weight held as bf16 or fp16
("QLoRA技术从入门到精通" §3(1): the FP16 base model is converted offline to
the 4-bit form).  The kernel widens each value exactly to fp32; the oracle
quantizes the exactly widened weight.  Indices, packed bytes, scale codes and
group constants are compared bit for bit, over every 16-bit value inside
blocks of several scales and on random weights."""

import numpy as np
import pytest

import workloads
from gpu_helpers import assert_quant_bit_exact, say
from oracle import nf4 as onf4
from oracle.bf16 import bits_to_float

pytestmark = pytest.mark.gpu


def _widen(bits, fmt):
    """uint16 patterns -> exact float32 values."""
    if fmt == "bf16":
        return bits_to_float(bits).astype(np.float32)
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float32)


def _device(bits, fmt):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if fmt == "bf16" else torch.float16).cuda()


def _every_value_blocks(fmt, scale_bits, per=63):
    """Blocks whose absmax is the 16-bit value `scale_bits`, together holding
    every finite 16-bit value of magnitude at most that (both signs)."""
    sign = np.uint16(0x8000)
    mag = np.arange(0, int(scale_bits) + 1, dtype=np.uint16)          # |v| <= scale: bit order = value order
    vals = np.concatenate([mag, mag[1:] | sign])
    nblk = -(-vals.size // per)
    B = np.zeros((nblk, 64), np.uint16)
    for b in range(nblk):
        chunk = vals[b * per:(b + 1) * per]
        B[b, 0] = scale_bits if b % 2 == 0 else (scale_bits | sign)
        B[b, 1:1 + chunk.size] = chunk
    return B.reshape(-1)


def _run(bits2d, fmt, table=0):
    import nf4_bit_quantized_amd as q
    import torch
    levels = None if table == 0 else onf4.uniform_levels()
    Q = onf4.quantize(_widen(bits2d, fmt), levels=levels)
    packed, codes, consts = q.qlora_quantize_nf4(_device(bits2d, fmt), table=table)
    torch.cuda.synchronize()
    assert_quant_bit_exact({"packed_h": packed.cpu().numpy(), "codes_h": codes.cpu().numpy(),
                            "consts_h": consts.cpu().numpy()}, Q)


def _scale_bits(fmt, x):
    if fmt == "bf16":
        return int(np.float32(x).view(np.uint32) >> 16)
    return int(np.float16(x).view(np.uint16))


@pytest.mark.parametrize("fmt,scales", [
    ("bf16", (1.0, 0.0123, 7.25)),
    ("bf16", (1.0e-30, 3.0e38)),
    ("fp16", (1.0, 0.0123, 7.25)),
    ("fp16", (6.0e-5, 65504.0)),        # a subnormal-range scale, the largest finite
])
def test_every_16bit_value_bit_exact(fmt, scales):
    parts = [_every_value_blocks(fmt, _scale_bits(fmt, s)) for s in scales]
    W = np.concatenate(parts)
    pad = (-W.size) % (64 * 64)
    W = np.concatenate([W, np.zeros(pad, np.uint16)]).reshape(64, -1)
    say(f"every {fmt} value, scales {scales}, W {W.shape}")
    _run(W, fmt)


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
@pytest.mark.parametrize("d_out,d_in", [(256, 256), (192, 320), (4096, 4096)])
def test_random_16bit_weight_bit_exact(fmt, d_out, d_in):
    say(f"random {fmt} weight {d_out}x{d_in}")
    W = workloads.layer_inputs(d_out, d_in, 1, 1, seed=50, with_dy=False)["W"]
    bits = workloads.bf16_bits(W) if fmt == "bf16" else W.astype(np.float16).view(np.uint16)
    _run(bits, fmt)


def test_16bit_weight_with_uniform_table():
    W = workloads.layer_inputs(256, 512, 1, 1, seed=51, with_dy=False)["W"]
    _run(workloads.bf16_bits(W), "bf16", table=1)
    _run(W.astype(np.float16).view(np.uint16), "fp16", table=1)


def test_16bit_weight_equals_fp32_path():
    """A bf16 weight gives the same bytes as its fp32 widening through the fp32 entry point."""
    import nf4_bit_quantized_amd as q
    import torch
    W = workloads.layer_inputs(512, 1024, 1, 1, seed=52, with_dy=False)["W"]
    bits = workloads.bf16_bits(W)
    a = q.qlora_quantize_nf4(_device(bits, "bf16"))
    b = q.qlora_quantize_nf4(torch.from_numpy(_widen(bits, "bf16")).cuda())
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
