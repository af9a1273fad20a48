"""GPU parity for the format without the second level: each block keeps its
fp32 absmax scale ("7、QLoRA 量化微调" §7.1, extended calculation: 64 weights
sharing one fp32 scale cost 4.5 bits per weight; double quantization is the
step that shrinks this).  The packed indices and the fp32 scales are
bit-exact against the oracle; the layer's products and both exports restore
with s'_b = s_b."""

import numpy as np
import pytest

import workloads
from gpu_helpers import TOL, dev_bf16, dev_f32, host_bf16_to_f64, normwise_err, oracle_layer, say
from oracle import nf4 as onf4
from oracle.bf16 import bits_to_float, float_to_bits

pytestmark = pytest.mark.gpu


def _check_quant(packed, codes, consts, Q):
    assert codes.numel() == 0
    np.testing.assert_array_equal(packed.cpu().numpy(), Q.packed)
    np.testing.assert_array_equal(consts.cpu().numpy().view(np.uint32), Q.scales.view(np.uint32))


@pytest.mark.parametrize("bs", [64, 256])
@pytest.mark.parametrize("d_out,d_in", [(256, 256), (64, 320), (4096, 4096)])
def test_quantize_bit_exact(bs, d_out, d_in):
    import nf4_bit_quantized_amd as q
    import torch
    say(f"fp32 scales bs={bs} {d_out}x{d_in}")
    W = workloads.layer_inputs(d_out, d_in, 1, 1, seed=90, with_dy=False)["W"]
    g = q.qlora_quantize_nf4(dev_f32(W), blocksize=bs, double_quant=False)
    bits = workloads.bf16_bits(W)
    h = q.qlora_quantize_nf4(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda(), blocksize=bs,
                             double_quant=False)
    torch.cuda.synchronize()
    _check_quant(*g, onf4.quantize(W, blocksize=bs, dq_blocksize=0))
    _check_quant(*h, onf4.quantize(bits_to_float(bits).astype(np.float32), blocksize=bs, dq_blocksize=0))


CASES = [
    # (d_out, d_in, T, r, alpha, seed, bs): at most 16 tokens take the few-token
    # kernel when rows hold whole blocks (the scales staged in LDS), else the tiles
    (256, 512, 4, 8, 16.0, 91, 64),
    (192, 320, 1, 16, 16.0, 92, 128),   # rows of 2.5 blocks: the tiles
    (192, 384, 1, 16, 16.0, 95, 128),   # 3 scales per row (odd), blocks of 128
    (128, 192, 2, 8, 16.0, 96, 64),     # 3 scales per row: a half chunk at the row's end
    (256, 1024, 16, 8, 16.0, 97, 256),  # 16 tokens, blocks of 256
    (256, 256, 100, 16, 32.0, 93, 64),
    (320, 448, 600, 24, 8.0, 94, 256),
]


@pytest.mark.parametrize("d_out,d_in,T,r,alpha,seed,bs", CASES)
def test_fwd_bwd_parity(d_out, d_in, T, r, alpha, seed, bs):
    import nf4_bit_quantized_amd as q
    import torch
    say(f"fp32 scales fwd/bwd bs={bs} d_out={d_out} d_in={d_in} T={T} r={r}")
    inp = workloads.layer_inputs(d_out, d_in, T, r, seed)
    Q = onf4.quantize(inp["W"], blocksize=bs, dq_blocksize=0)
    o = oracle_layer(inp, r, alpha, Q=Q)
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]), blocksize=bs, double_quant=False)
    X, A, B, dY = (dev_bf16(inp[k]) for k in ("X", "A", "B", "dY"))
    q.qlora_trace_select({"decode"})
    q.qlora_trace_read(reset=True)
    try:
        Y, U = q.qlora_linear_fwd(packed, codes, consts, X, A, B, alpha)
        torch.cuda.synchronize()
        decode_launches = q.qlora_trace_read(reset=True).get("decode", (0, 0.0))[0]
    finally:
        q.qlora_trace_enable(False)
    # the few-token kernel takes the call exactly when rows hold whole blocks
    assert decode_launches == (1 if T <= 16 and d_in % bs == 0 else 0), decode_launches
    dX, dA, dB = q.qlora_linear_bwd(packed, codes, consts, X, A, B, alpha, dY, U_in=U)
    torch.cuda.synchronize()
    _check_quant(packed, codes, consts, Q)
    got = {"Y": host_bf16_to_f64(Y), "U": U.cpu().numpy().astype(np.float64), "dX": host_bf16_to_f64(dX),
           "dA": dA.cpu().numpy().astype(np.float64), "dB": dB.cpu().numpy().astype(np.float64)}
    errs = {k: normwise_err(got[k], o[k]) for k in got}
    say("  errors", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= TOL, (k, v)


@pytest.mark.parametrize("bs", [64, 128])
def test_exports(bs):
    import nf4_bit_quantized_amd as q
    import torch
    from oracle import lora as olora
    d_out, d_in, r, alpha = 192, 4160, 16, 16.0
    inp = workloads.layer_inputs(d_out, d_in, 1, r, seed=95)
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]), blocksize=bs, double_quant=False)
    Wh = q.qlora_dequantize_nf4(packed, codes, consts)
    Wm = q.qlora_merge_lora(packed, codes, consts, dev_bf16(inp["A"]), dev_bf16(inp["B"]), alpha)
    torch.cuda.synchronize()
    W_hat = onf4.dequantize(onf4.quantize(inp["W"], blocksize=bs, dq_blocksize=0))
    np.testing.assert_array_equal(Wh.view(torch.int16).cpu().numpy().view(np.uint16), float_to_bits(W_hat))
    want = olora.merged_weight(W_hat, bits_to_float(inp["A"]), bits_to_float(inp["B"]), alpha, r)
    got = host_bf16_to_f64(Wm)
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 7)
    tol = step + 2.0 ** -20 * (np.abs(W_hat) + np.abs(want - W_hat))
    assert float(np.max(np.abs(got - want) / tol)) <= 1.0
    # the restored weight differs from the double-quantized format's (s' = s_b here)
    p2, c2, k2 = q.qlora_quantize_nf4(dev_f32(inp["W"]), blocksize=bs)
    W2 = q.qlora_dequantize_nf4(p2, c2, k2)
    torch.cuda.synchronize()
    assert not torch.equal(W2.view(torch.int16), Wh.view(torch.int16))


@pytest.mark.parametrize("d_out,d_in", [(28672, 8192), (8192, 28672)])
def test_decode_shapes_full_size_sampled(d_out, d_in):
    """The few-token forward in this format at the decode shapes, T = 1, 4
    and 16, r = 64, alpha = 16, on the weight-streaming kernel (one `decode`
    launch per call): Y on 48 sampled output columns against the oracle
    (normwise, and per element within the kernel's rounding bound), the
    sampled rows' packed bytes and fp32 scales bit-exact.  Without the second level every 64-weight block of a
    row is quantized on its own, so the oracle quantizes just those rows."""
    import nf4_bit_quantized_amd as q
    import torch
    from gpu_helpers import elementwise_stats
    from oracle import lora as olora
    r, alpha = 64, 16.0
    say(f"fp32 scales decode shape {d_out}x{d_in}: drawing inputs")
    inp = workloads.layer_inputs(d_out, d_in, 16, r, seed=6, with_dy=False)
    rng = np.random.default_rng(d_out + 3 * d_in)
    rows = np.sort(rng.choice(d_out, size=48, replace=False))
    Q = onf4.quantize(inp["W"][rows], dq_blocksize=0)
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]), double_quant=False)
    assert codes.numel() == 0
    nb = d_in // 64
    np.testing.assert_array_equal(packed[torch.as_tensor(rows, device="cuda")].cpu().numpy(),
                                  Q.packed.reshape(len(rows), d_in // 2))
    np.testing.assert_array_equal(consts.view(d_out, nb)[torch.as_tensor(rows, device="cuda")].cpu().numpy()
                                  .view(np.uint32), Q.scales.reshape(len(rows), nb).view(np.uint32))
    say("  sampled rows bit-exact")
    W_rows = onf4.dequantize(Q).astype(np.float64)
    X = bits_to_float(inp["X"])
    A, B = bits_to_float(inp["A"]), bits_to_float(inp["B"])
    Ag, Bg = dev_bf16(inp["A"]), dev_bf16(inp["B"])
    ri = torch.as_tensor(rows, device="cuda")
    for T in (1, 4, 16):
        Xg = dev_bf16(inp["X"][:T])
        q.qlora_trace_select({"decode"})
        q.qlora_trace_read(reset=True)
        try:
            Y, _ = q.qlora_linear_fwd(packed, codes, consts, Xg, Ag, Bg, alpha)
            torch.cuda.synchronize()
            assert q.qlora_trace_read(reset=True).get("decode", (0, 0.0))[0] == 1
        finally:
            q.qlora_trace_enable(False)
        got = host_bf16_to_f64(Y.index_select(1, ri))
        want, _ = olora.forward(W_rows, X[:T], A, B[rows], alpha, r)
        # per element: this kernel scales each block's products by s' in fp32
        # instead of rounding T[q] * s' to bf16 first, one bf16 rounding (2^-8)
        # per weight; with the output's own rounding the error stays within
        # 2^-8 |Y| + 2^-7 (sum of the terms' magnitudes), which the oracle gives
        # on absolute values
        mag, _ = olora.forward(np.abs(W_rows), np.abs(X[:T]), np.abs(A), np.abs(B[rows]), alpha, r)
        worst = float(np.max(np.abs(got - want) / (2.0 ** -8 * np.abs(want) + 2.0 ** -7 * mag)))
        err, st = normwise_err(got, want), elementwise_stats(got, want)
        say(f"  T={T}: normwise {err:.2e}, elementwise {st}, rounding-bound ratio {worst:.3f}")
        assert err <= TOL
        assert worst <= 1.0
