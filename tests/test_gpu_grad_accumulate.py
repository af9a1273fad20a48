"""Gradient accumulation of the adapter gradients over micro-batches ("LoRA 与
QLoRA：把大模型微调拆成可负担的工程" §10: accumulation simulates a larger
effective batch): qlora_linear_bwd_accumulate adds s G^T X and s dY^T U to
what dA and dB hold.  Checked bit for bit against fl32(old + the overwriting
call's result), and against the oracle's float64 sum over the micro-batches."""

import numpy as np
import pytest

import workloads
from gpu_helpers import TOL, dev_bf16, dev_f32, normwise_err, oracle_layer, say
from oracle import nf4 as onf4

pytestmark = pytest.mark.gpu

# (d_out, d_in, T, r): streaming adapter kernels (many tokens, r % 8 == 0, r <= 64),
# and the split-contraction ones (few tokens, odd rank, rank above 64)
ACC_CASES = [(256, 320, 600, 16), (192, 256, 8, 8), (320, 192, 100, 3), (256, 256, 40, 128)]


@pytest.mark.parametrize("d_out,d_in,T,r", ACC_CASES)
def test_accumulate_adds_to_the_given_gradients(d_out, d_in, T, r):
    import nf4_bit_quantized_amd as q
    import torch
    alpha = 16.0
    say(f"accumulate {d_out}x{d_in} T={T} r={r}")
    inp = workloads.layer_inputs(d_out, d_in, T, r, seed=60)
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]))
    X, A, B, dY = (dev_bf16(inp[k]) for k in ("X", "A", "B", "dY"))
    _, U = q.qlora_linear_fwd(packed, codes, consts, X, A, B, alpha)
    dX0, dA_new, dB_new = q.qlora_linear_bwd(packed, codes, consts, X, A, B, alpha, dY, U_in=U)
    g = torch.Generator().manual_seed(61)
    dA0 = torch.randn((r, d_in), generator=g).cuda()
    dB0 = torch.randn((d_out, r), generator=g).cuda()
    dA, dB = dA0.clone(), dB0.clone()
    dX1, _, _ = q.qlora_linear_bwd(packed, codes, consts, X, A, B, alpha, dY, U_in=U, dA=dA, dB=dB,
                                   accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(dA, dA0 + dA_new)
    assert torch.equal(dB, dB0 + dB_new)
    assert torch.equal(dX1.view(torch.int16), dX0.view(torch.int16))


@pytest.mark.parametrize("d_out,d_in,T,r", [(256, 320, 600, 16), (320, 192, 12, 3)])
def test_accumulate_over_micro_batches_matches_oracle(d_out, d_in, T, r):
    """Three micro-batches (different X and dY, same weight and adapter),
    accumulated from zero, against the oracle's summed float64 gradients."""
    import nf4_bit_quantized_amd as q
    import torch
    alpha = 8.0
    say(f"micro-batches {d_out}x{d_in} T={T} r={r}")
    base = workloads.layer_inputs(d_out, d_in, T, r, seed=62)
    Q = onf4.quantize(base["W"])
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(base["W"]))
    A, B = dev_bf16(base["A"]), dev_bf16(base["B"])
    dA = torch.zeros((r, d_in), dtype=torch.float32, device="cuda")
    dB = torch.zeros((d_out, r), dtype=torch.float32, device="cuda")
    want_A = np.zeros((r, d_in))
    want_B = np.zeros((d_out, r))
    for mb in range(3):
        step = workloads.layer_inputs(d_out, d_in, T, r, seed=63 + mb)
        inp = dict(base, X=step["X"], dY=step["dY"])
        o = oracle_layer(inp, r, alpha, Q=Q)
        want_A += o["dA"]
        want_B += o["dB"]
        X, dY = dev_bf16(inp["X"]), dev_bf16(inp["dY"])
        q.qlora_linear_bwd(packed, codes, consts, X, A, B, alpha, dY, dA=dA, dB=dB, want_dx=False,
                           accumulate=True)
    torch.cuda.synchronize()
    eA = normwise_err(dA.cpu().numpy().astype(np.float64), want_A)
    eB = normwise_err(dB.cpu().numpy().astype(np.float64), want_B)
    say(f"  dA {eA:.2e} dB {eB:.2e}")
    assert eA <= TOL and eB <= TOL


def test_accumulate_with_no_tokens_leaves_gradients():
    import nf4_bit_quantized_amd as q
    import torch
    inp = workloads.layer_inputs(128, 128, 1, 8, seed=64)
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]))
    A, B = dev_bf16(inp["A"]), dev_bf16(inp["B"])
    X = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    dY = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    dA = torch.full((8, 128), 3.0, device="cuda")
    dB = torch.full((128, 8), -2.0, device="cuda")
    q.qlora_linear_bwd(packed, codes, consts, X, A, B, 4.0, dY, dA=dA, dB=dB, accumulate=True)
    q.qlora_linear_bwd(packed, codes, consts, X, A, B, 4.0, dY)
    torch.cuda.synchronize()
    assert bool((dA == 3.0).all()) and bool((dB == -2.0).all())
