"""GPU parity of the dX product on 256 x 256 tiles (the multiplying waves
restore each step's weight rows into LDS and read them back transposed),
which the library takes when its rounds of the GPU cost no more than the
256 x 128 kernel's (e.g. 512 tiles).  The shapes below reach that count
with short contractions (few weight rows), so the oracle stays cheap;
they cover ragged token tiles and a last output tile 64 wide, contractions of 2, 3, 4, 7, 8 and 16 steps (the loop's pairs and its
odd end), ranks that are and are not multiples of 8, rank 0, blocks of 128
and 256, fp32 block scales and the uniform table.  dX is compared with the
oracle (normwise bar and elementwise statistics), dA and dB too; through
one-hot rows of dY every output must be one restored weight, bit for bit;
the product over several weights (their rows one contraction) and its
layer-by-layer form (dX rounded after each layer and accumulated) are
compared with the oracle's sum; a shape whose last round of wide tiles
would be nearly empty runs whole rounds wide and its last columns on the
256 x 128 kernel (through that kernel's weight-column offset), checked the
same ways."""

import numpy as np
import pytest

import workloads
from gpu_helpers import (TOL, dev_bf16, dev_f32, elementwise_stats, host_bf16_to_f64, normwise_err,
                         oracle_sampled, rounding_bound_ratio, say)
from oracle import lora as olora
from oracle import nf4 as onf4
from oracle.bf16 import bits_to_float

pytestmark = pytest.mark.gpu

# (d_out, d_in, T, r, alpha, seed, blocksize, double_quant, table)
WIDE_DX = [
    (128, 32768, 1000, 8, 16.0, 60, 64, True, 0),      # 4 x 128 tiles, last token tile 232 rows, 2 steps
    (448, 32576, 1000, 12, 24.0, 61, 64, True, 0),     # 4 x 128 tiles, last output tile 64 wide, 7 steps
    (256, 32768, 1024, 16, 32.0, 62, 128, False, 0),   # fp32 block scales, blocks of 128, 4 steps
    (192, 65536, 512, 0, 0.0, 63, 64, True, 0),        # base branch only, 3 steps
    (512, 32768, 1024, 64, 16.0, 64, 64, True, 1),     # uniform table, r = 64 (two tail steps), 8 steps
    (1024, 16384, 2048, 3, 6.0, 65, 256, True, 0),     # blocks of 256, odd rank, 16 steps
]


@pytest.mark.parametrize("d_out,d_in,T,r,alpha,seed,bs,dq,table", WIDE_DX)
def test_wide_dx_matches_oracle(d_out, d_in, T, r, alpha, seed, bs, dq, table):
    import torch
    import nf4_bit_quantized_amd as q
    say(f"wide dX d_out={d_out} d_in={d_in} T={T} r={r} bs={bs} dq={dq} table={table}")
    assert ((T + 255) // 256) * ((d_in + 255) // 256) == 512
    inp = workloads.layer_inputs(d_out, d_in, T, r, seed)
    levels = onf4.uniform_levels() if table == 1 else None
    Q = onf4.quantize(inp["W"], levels=levels, blocksize=bs, dq_blocksize=256 if dq else 0)
    W_hat = onf4.dequantize(Q, levels=levels).astype(np.float64)
    X = bits_to_float(inp["X"])
    A = bits_to_float(inp["A"]) if r else None
    B = bits_to_float(inp["B"]) if r else None
    dXo, dAo, dBo = olora.backward(W_hat, X, A, B, bits_to_float(inp["dY"]), alpha, r)

    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]), table=table, blocksize=bs, double_quant=dq)
    dX, dA, dB = q.qlora_linear_bwd(packed, codes, consts, dev_bf16(inp["X"]), dev_bf16(inp["A"]) if r else None,
                                    dev_bf16(inp["B"]) if r else None, alpha, dev_bf16(inp["dY"]), table=table)
    torch.cuda.synchronize()
    dXg = host_bf16_to_f64(dX)
    err = normwise_err(dXg, dXo)
    st = elementwise_stats(dXg, dXo)
    say(f"  dX normwise {err:.2e}, elementwise {st}")
    assert err <= TOL
    # a local fault (a wrong block, a wrong tail row, a misplaced column) shows as large elementwise errors
    assert st["share_above_1e-2"] < 1e-3
    if r:
        assert normwise_err(dA.cpu().numpy(), dAo) <= TOL
        assert normwise_err(dB.cpu().numpy(), dBo) <= TOL


@pytest.mark.parametrize("d_out,d_in,bs,dq,table", [(256, 32768, 64, True, 0), (128, 65536, 128, False, 1)])
def test_wide_dx_restore_bit_exact_through_one_hot_rows(d_out, d_in, bs, dq, table):
    """Row t of dY is the one-hot row of weight row t mod d_out, r = 0:
    dX[t][k] is the single product 1 * W_hat[t mod d_out][k], so dX must equal
    the oracle's restored weight bit for bit (every column in its place)."""
    import torch
    import nf4_bit_quantized_amd as q
    T = 1024 if d_in == 32768 else 512
    say(f"wide dX one-hot d_out={d_out} d_in={d_in} T={T} bs={bs} dq={dq} table={table}")
    inp = workloads.layer_inputs(d_out, d_in, 1, 1, seed=66, with_dy=False)
    levels = onf4.uniform_levels() if table == 1 else None
    W_hat = onf4.dequantize(onf4.quantize(inp["W"], levels=levels, blocksize=bs, dq_blocksize=256 if dq else 0),
                            levels=levels)
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]), table=table, blocksize=bs, double_quant=dq)
    rows = np.arange(T) % d_out
    dY = torch.zeros((T, d_out), dtype=torch.bfloat16, device="cuda")
    dY[torch.arange(T, device="cuda"), torch.from_numpy(rows).cuda()] = 1.0
    X = torch.zeros((T, d_in), dtype=torch.bfloat16, device="cuda")
    dX, _, _ = q.qlora_linear_bwd(packed, codes, consts, X, None, None, 0.0, dY, table=table)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dX.float().cpu().numpy(), W_hat[rows])


def _layers(shapes, K, T, r, seed, tables):
    import nf4_bit_quantized_amd as q
    X = workloads.layer_inputs(64, K, T, 1, seed, with_dy=False)["X"]
    out = []
    for i, N in enumerate(shapes):
        inp = workloads.layer_inputs(N, K, T, r, seed + 1 + i)
        pk, cd, cs = q.qlora_quantize_nf4(dev_f32(inp["W"]), table=tables[i])
        out.append(dict(inp=inp, dev=(pk, cd, cs, dev_bf16(inp["A"]) if r else None, dev_bf16(inp["B"]) if r else None),
                        levels=None if tables[i] == 0 else onf4.uniform_levels()))
    return X, out


@pytest.mark.parametrize("shapes,r,tables", [
    ((192, 64, 128), 8, (0, 0, 0)),       # one product over three weights' rows, then their tails
    ((128, 256), 12, (0, 0)),             # two weights, rank not a multiple of 8
    ((64, 64, 64, 128), 0, (0, 0, 0, 0)),  # four weights, no tails
    ((128, 192), 8, (1, 0)),              # different tables: layer by layer, dX accumulated
])
def test_wide_dx_over_several_weights(shapes, r, tables):
    import torch
    import nf4_bit_quantized_amd as q
    K, T, alpha = 32768, 1024, 16.0
    say(f"wide dX several weights shapes={shapes} r={r} tables={tables}")
    Xb, layers = _layers(shapes, K, T, r, 170, list(tables))
    X = dev_bf16(Xb)
    dYs = [dev_bf16(l["inp"]["dY"]) for l in layers]
    dX, grads = q.qlora_linear_bwd_multi([l["dev"] for l in layers], X, alpha, dYs, tables=list(tables))
    torch.cuda.synchronize()
    Xf = bits_to_float(Xb)
    want, mag = 0.0, 0.0
    for l, (dA, dB) in zip(layers, grads):
        W_hat = onf4.dequantize(onf4.quantize(l["inp"]["W"], levels=l["levels"]), levels=l["levels"])
        A = bits_to_float(l["inp"]["A"]) if r else None
        B = bits_to_float(l["inp"]["B"]) if r else None
        dXo, dAo, dBo = olora.backward(W_hat, Xf, A, B, bits_to_float(l["inp"]["dY"]), alpha, r)
        want = want + dXo
        # the layer's dX on absolute values: a bound on the magnitudes of its terms
        mag = mag + olora.backward(np.abs(W_hat), np.abs(Xf), None if A is None else np.abs(A),
                                   None if B is None else np.abs(B), np.abs(bits_to_float(l["inp"]["dY"])),
                                   alpha, r)[0]
        if r:
            assert normwise_err(dA.cpu().numpy(), dAo) <= TOL
            assert normwise_err(dB.cpu().numpy(), dBo) <= TOL
    got = host_bf16_to_f64(dX)
    err = normwise_err(got, want)
    st = elementwise_stats(got, want)
    say(f"  dX normwise {err:.2e}, elementwise {st}")
    assert err <= TOL
    if len(set(tables)) == 1:
        # one product: dX is one fp32 sum, rounded once
        assert st["share_above_1e-2"] < 1e-3
    else:
        # layer by layer: each layer's dX is rounded to bf16 and added to the
        # rounded sum so far, so an element whose parts nearly cancel keeps an
        # error of a bf16 step of its parts; every element stays within 2^-8
        # of |dX| plus 2^-8 of the magnitudes of its terms
        ratio = rounding_bound_ratio(got, want, mag, 2.0 ** -8)
        say(f"  rounding bound ratio {ratio:.3f}")
        assert ratio <= 1.0


def test_wide_and_tiled_dx_agree_on_a_training_shape():
    """At 4096 tokens and 8192 x 8192 dX runs on 256 x 256 tiles; the same
    backward split into four calls of 1024 tokens (128 tiles each: the
    256 x 128 kernel) must agree with it to within fp32 accumulation order,
    and both with the oracle on sampled columns."""
    import torch
    import nf4_bit_quantized_amd as q
    d_out = d_in = 8192
    T, r, alpha = 4096, 64, 16.0
    say("wide vs tiled dX 8192x8192 T=4096")
    g = torch.Generator(device="cuda").manual_seed(67)
    W = torch.randn(d_out, d_in, device="cuda", generator=g) * 0.02
    X = torch.randn(T, d_in, device="cuda", generator=g).to(torch.bfloat16)
    dY = torch.randn(T, d_out, device="cuda", generator=g).to(torch.bfloat16)
    A = (torch.randn(r, d_in, device="cuda", generator=g) / r).to(torch.bfloat16)
    B = (torch.randn(d_out, r, device="cuda", generator=g) * 0.01).to(torch.bfloat16)
    packed, codes, consts = q.qlora_quantize_nf4(W)
    dXw, _, _ = q.qlora_linear_bwd(packed, codes, consts, X, A, B, alpha, dY)
    dXt = torch.cat([q.qlora_linear_bwd(packed, codes, consts, X[i:i + 1024].contiguous(), A, B, alpha,
                                        dY[i:i + 1024].contiguous())[0] for i in range(0, T, 1024)])
    torch.cuda.synchronize()
    d = (dXw.float() - dXt.float()).abs().max().item()
    scale = dXt.float().abs().max().item()
    say(f"  max |wide - tiled| = {d:.3e} (max |dX| {scale:.3e})")
    assert d <= 2 ** -7 * scale
    # sampled columns (one per 64-column block position and tile edge) against the oracle
    cols = np.array([0, 1, 7, 8, 63, 64, 255, 256, 1000, 4095, 4096, 8191])
    Q = onf4.quantize(W.cpu().numpy())
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    o = oracle_sampled(Q, f64(X), f64(A), f64(B), f64(dY), alpha, r, rows=np.array([0]), cols=cols)
    got = f64(dXw[:, cols])
    err = normwise_err(got, o["dX"])
    say(f"  sampled columns normwise {err:.2e}, elementwise {elementwise_stats(got, o['dX'])}")
    assert err <= TOL


# d_in = 33216 at 1024 tokens: 4 x 130 tiles of 256 x 256, two full rounds of
# the GPU plus 8 tiles; the wide launch keeps the 128 tile columns of the two
# rounds and the 256 x 128 kernel takes the last 448 columns (the weight's
# columns 32768 .. 33215, through its column offset).
SPLIT_K = 33216


@pytest.mark.parametrize("d_out,T,r,alpha,seed", [(128, 1024, 8, 16.0, 70), (192, 1000, 12, 24.0, 71)])
def test_wide_dx_with_a_narrow_last_round_matches_oracle(d_out, T, r, alpha, seed):
    import torch
    import nf4_bit_quantized_amd as q
    say(f"wide dX + narrow tail d_out={d_out} d_in={SPLIT_K} T={T} r={r}")
    inp = workloads.layer_inputs(d_out, SPLIT_K, T, r, seed)
    W_hat = onf4.dequantize(onf4.quantize(inp["W"])).astype(np.float64)
    dXo, dAo, dBo = olora.backward(W_hat, bits_to_float(inp["X"]), bits_to_float(inp["A"]),
                                   bits_to_float(inp["B"]), bits_to_float(inp["dY"]), alpha, r)
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]))
    dX, dA, dB = q.qlora_linear_bwd(packed, codes, consts, dev_bf16(inp["X"]), dev_bf16(inp["A"]),
                                    dev_bf16(inp["B"]), alpha, dev_bf16(inp["dY"]))
    torch.cuda.synchronize()
    got = host_bf16_to_f64(dX)
    err = normwise_err(got, dXo)
    st = elementwise_stats(got, dXo)
    tail = elementwise_stats(got[:, 32768:], dXo[:, 32768:])
    say(f"  dX normwise {err:.2e}, elementwise {st}, last 448 columns {tail}")
    assert err <= TOL
    assert st["share_above_1e-2"] < 1e-3 and tail["share_above_1e-2"] < 1e-3
    assert normwise_err(dA.cpu().numpy(), dAo) <= TOL
    assert normwise_err(dB.cpu().numpy(), dBo) <= TOL


def test_wide_dx_with_a_narrow_last_round_bit_exact_through_one_hot_rows():
    """As test_wide_dx_restore_bit_exact_through_one_hot_rows, at the split
    shape: every column of both launches, the narrow one's included, holds
    the restored weight of its own column."""
    import torch
    import nf4_bit_quantized_amd as q
    d_out, T = 128, 1024
    say(f"wide dX + narrow tail one-hot d_out={d_out} d_in={SPLIT_K} T={T}")
    inp = workloads.layer_inputs(d_out, SPLIT_K, 1, 1, seed=72, with_dy=False)
    W_hat = onf4.dequantize(onf4.quantize(inp["W"]))
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]))
    rows = np.arange(T) % d_out
    dY = torch.zeros((T, d_out), dtype=torch.bfloat16, device="cuda")
    dY[torch.arange(T, device="cuda"), torch.from_numpy(rows).cuda()] = 1.0
    X = torch.zeros((T, SPLIT_K), dtype=torch.bfloat16, device="cuda")
    dX, _, _ = q.qlora_linear_bwd(packed, codes, consts, X, None, None, 0.0, dY)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dX.float().cpu().numpy(), W_hat[rows])


def test_wide_dx_with_a_narrow_last_round_over_several_weights():
    import torch
    import nf4_bit_quantized_amd as q
    shapes, r, T, alpha = (128, 64), 8, 1024, 16.0
    say(f"wide dX + narrow tail several weights shapes={shapes} d_in={SPLIT_K}")
    Xb, layers = _layers(shapes, SPLIT_K, T, r, 180, [0, 0])
    dX, grads = q.qlora_linear_bwd_multi([l["dev"] for l in layers], dev_bf16(Xb), alpha,
                                         [dev_bf16(l["inp"]["dY"]) for l in layers])
    torch.cuda.synchronize()
    Xf = bits_to_float(Xb)
    want = 0.0
    for l in layers:
        W_hat = onf4.dequantize(onf4.quantize(l["inp"]["W"]))
        want = want + olora.backward(W_hat, Xf, bits_to_float(l["inp"]["A"]), bits_to_float(l["inp"]["B"]),
                                     bits_to_float(l["inp"]["dY"]), alpha, r)[0]
    got = host_bf16_to_f64(dX)
    err = normwise_err(got, want)
    st = elementwise_stats(got, want)
    say(f"  dX normwise {err:.2e}, elementwise {st}")
    assert err <= TOL
    assert st["share_above_1e-2"] < 1e-3
