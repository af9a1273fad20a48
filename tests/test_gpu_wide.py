"""GPU parity of the forward product on 256 x 256 tiles (the restore in the
multiplying waves' registers), which the library takes when its rounds of
the GPU cost no more than the 256 x 128 kernel's (e.g. 512 tiles).  The
shapes below reach that count with short contractions, so the oracle stays
cheap; they cover ragged token and output
tiles, contractions of 2, 3, 7 and 8 steps (the pipelined loop and its ends),
ranks that are and are not multiples of 8, rank 0, blocks of 128, fp32 block
scales and the uniform table.  Y is compared with the oracle (normwise bar
and elementwise statistics), U with the oracle, quantization bit-exact, and
through one-hot token rows every output must be one restored weight,
bit for bit."""

import numpy as np
import pytest

import workloads
from gpu_helpers import (TOL, assert_quant_bit_exact, dev_bf16, dev_f32, elementwise_stats, host_bf16_to_f64,
                         normwise_err, say)
from oracle import lora as olora
from oracle import nf4 as onf4
from oracle.bf16 import bits_to_float

pytestmark = pytest.mark.gpu

# (d_out, d_in, T, r, alpha, seed, blocksize, double_quant, table)
WIDE = [
    (32768, 128, 1000, 8, 16.0, 40, 64, True, 0),       # 4 x 128 tiles, last token tile 232 rows, 2 steps
    (32576, 448, 1000, 12, 24.0, 41, 64, True, 0),      # 4 x 128 tiles, last output tile 64 wide, r % 8 != 0
    (32768, 256, 1024, 16, 32.0, 42, 128, False, 0),    # fp32 block scales, blocks of 128
    (65536, 192, 512, 0, 0.0, 43, 64, True, 0),         # base branch only, 3 steps
    (32768, 512, 1024, 64, 16.0, 44, 64, True, 1),      # uniform table, r = 64, 8 steps
    (16384, 1024, 2048, 3, 6.0, 45, 256, True, 0),      # blocks of 256, odd rank, 16 steps
]


@pytest.mark.parametrize("d_out,d_in,T,r,alpha,seed,bs,dq,table", WIDE)
def test_wide_forward_matches_oracle(d_out, d_in, T, r, alpha, seed, bs, dq, table):
    import torch
    import nf4_bit_quantized_amd as q
    say(f"wide fwd d_out={d_out} d_in={d_in} T={T} r={r} bs={bs} dq={dq} table={table}")
    assert ((T + 255) // 256) * ((d_out + 255) // 256) == 512
    inp = workloads.layer_inputs(d_out, d_in, T, r, seed, with_dy=False)
    levels = onf4.uniform_levels() if table == 1 else None
    Q = onf4.quantize(inp["W"], levels=levels, blocksize=bs, dq_blocksize=256 if dq else 0)
    W_hat = onf4.dequantize(Q, levels=levels).astype(np.float64)
    X = bits_to_float(inp["X"])
    A = bits_to_float(inp["A"]) if r else None
    B = bits_to_float(inp["B"]) if r else None
    Yo, Uo = olora.forward(W_hat, X, A, B, alpha, r)

    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]), table=table, blocksize=bs, double_quant=dq)
    Y, U = q.qlora_linear_fwd(packed, codes, consts, dev_bf16(inp["X"]), dev_bf16(inp["A"]) if r else None,
                              dev_bf16(inp["B"]) if r else None, alpha, table=table)
    torch.cuda.synchronize()
    g = {"packed_h": packed.cpu().numpy(), "codes_h": codes.cpu().numpy(), "consts_h": consts.cpu().numpy()}
    if dq:
        assert_quant_bit_exact(g, Q)
    else:
        np.testing.assert_array_equal(g["packed_h"], Q.packed)
        np.testing.assert_array_equal(g["consts_h"].view(np.uint32), Q.scales.view(np.uint32))
    Yg = host_bf16_to_f64(Y)
    err = normwise_err(Yg, Yo)
    st = elementwise_stats(Yg, Yo)
    say(f"  Y normwise {err:.2e}, elementwise {st}")
    assert err <= TOL
    # a local fault (a wrong block, a wrong tail column) would show as a share of large elementwise errors
    assert st["share_above_1e-2"] < 1e-3
    if r:
        assert normwise_err(U.cpu().numpy(), Uo) <= 1e-5


@pytest.mark.parametrize("d_out,d_in,bs,dq,table", [(65536, 256, 64, True, 0), (32768, 512, 128, False, 1)])
def test_wide_restore_bit_exact_through_one_hot_rows(d_out, d_in, bs, dq, table):
    """Token t is the one-hot row of column t mod d_in, r = 0: Y[t][n] is the
    single product 1 * W_hat[n][t mod d_in], so Y must equal the oracle's
    restored weight bit for bit."""
    import torch
    import nf4_bit_quantized_amd as q
    T = 512 if d_out >= 65536 else 1024
    say(f"wide one-hot d_out={d_out} d_in={d_in} T={T} bs={bs} dq={dq} table={table}")
    inp = workloads.layer_inputs(d_out, d_in, 1, 1, seed=46, with_dy=False)
    levels = onf4.uniform_levels() if table == 1 else None
    W_hat = onf4.dequantize(onf4.quantize(inp["W"], levels=levels, blocksize=bs, dq_blocksize=256 if dq else 0),
                            levels=levels)
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]), table=table, blocksize=bs, double_quant=dq)
    cols = np.arange(T) % d_in
    X = torch.zeros((T, d_in), dtype=torch.bfloat16, device="cuda")
    X[torch.arange(T, device="cuda"), torch.from_numpy(cols).cuda()] = 1.0
    Y, _ = q.qlora_linear_fwd(packed, codes, consts, X, None, None, 0.0, table=table)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(Y.float().cpu().numpy(), W_hat.T[cols])


def test_wide_and_tiled_forward_agree_on_a_training_shape():
    """At 4096 tokens and 8192 x 8192 the wide kernel runs; the same layer
    split into four calls of 1024 tokens (256 tiles each: the 256 x 128
    kernel) must agree with it to within fp32 accumulation order, and both
    with the oracle on sampled rows."""
    import torch
    import nf4_bit_quantized_amd as q
    d_out = d_in = 8192
    T, r, alpha = 4096, 64, 16.0
    say("wide vs tiled 8192x8192 T=4096")
    g = torch.Generator(device="cuda").manual_seed(47)
    W = torch.randn(d_out, d_in, device="cuda", generator=g) * 0.02
    X = torch.randn(T, d_in, device="cuda", generator=g).to(torch.bfloat16)
    A = (torch.randn(r, d_in, device="cuda", generator=g) / r).to(torch.bfloat16)
    B = (torch.randn(d_out, r, device="cuda", generator=g) * 0.01).to(torch.bfloat16)
    packed, codes, consts = q.qlora_quantize_nf4(W)
    Yw, _ = q.qlora_linear_fwd(packed, codes, consts, X, A, B, alpha)
    Yt = torch.cat([q.qlora_linear_fwd(packed, codes, consts, X[i:i + 1024].contiguous(), A, B, alpha)[0]
                    for i in range(0, T, 1024)])
    torch.cuda.synchronize()
    d = (Yw.float() - Yt.float()).abs().max().item()
    scale = Yt.float().abs().max().item()
    say(f"  max |wide - tiled| = {d:.3e} (max |Y| {scale:.3e})")
    assert d <= 2 ** -7 * scale
    # sampled rows against the oracle
    rows = np.array([0, 1, 255, 256, 1023, 2048, 3071, 4095])
    Q = onf4.quantize(W.cpu().numpy())
    W_hat = onf4.dequantize(Q).astype(np.float64)
    Xr = X[rows].float().cpu().numpy().astype(np.float64)
    Yo, _ = olora.forward(W_hat, Xr, A.float().cpu().numpy().astype(np.float64),
                          B.float().cpu().numpy().astype(np.float64), alpha, r)
    Yg = Yw[rows].float().cpu().numpy().astype(np.float64)
    err = normwise_err(Yg, Yo)
    say(f"  sampled rows normwise {err:.2e}, elementwise {elementwise_stats(Yg, Yo)}")
    assert err <= TOL
