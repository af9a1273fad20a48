"""The allocation-free forward (qlora_linear_fwd_noalloc) against the forward
that takes a caller workspace (qlora_linear_fwd): the same kernels, so the
outputs must agree bit for bit -- two calls in a row, the second smaller, at
a many-token shape (tiled product, streamed rank-r pass) and at a few-token
shape (weight-streaming kernel, split rank-r pass), through the C ABI.
Also: a call beyond the static scratch is refused before any launch."""

import numpy as np
import pytest

import workloads
from gpu_helpers import dev_bf16, dev_f32, say

pytestmark = pytest.mark.gpu


def _layer(d_out, d_in, T, r, seed):
    import nf4_bit_quantized_amd as q
    inp = workloads.layer_inputs(d_out, d_in, T, r, seed, with_dy=False)
    packed, codes, consts = q.qlora_quantize_nf4(dev_f32(inp["W"]))
    return packed, codes, consts, dev_bf16(inp["X"]), dev_bf16(inp["A"]), dev_bf16(inp["B"])


@pytest.mark.parametrize("first,second", [
    ((1024, 2048, 1536, 64), (512, 1024, 300, 16)),     # many tokens (streamed, then split rank-r pass)
    ((2048, 4096, 16, 64), (1024, 1024, 3, 8)),          # few tokens, then fewer
])
def test_noalloc_forward_matches_workspace_forward(first, second):
    import torch
    import nf4_bit_quantized_amd as q
    for i, (d_out, d_in, T, r) in enumerate((first, second)):
        say(f"noalloc fwd call {i}: d_out {d_out} d_in {d_in} T {T} r {r}")
        packed, codes, consts, X, A, B = _layer(d_out, d_in, T, r, seed=10 + i)
        alpha = 16.0
        Y_ref, U_ref = q.qlora_linear_fwd(packed, codes, consts, X, A, B, alpha)
        Y = torch.full((T, d_out), float("nan"), dtype=torch.bfloat16, device="cuda")
        U = torch.full((T, r), float("nan"), dtype=torch.float32, device="cuda")
        q.qlora_linear_fwd_noalloc(packed, codes, consts, X, A, B, alpha, Y, U_out=U)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), Y_ref.view(torch.int16)), "Y differs"
        assert torch.equal(U.view(torch.int32), U_ref.view(torch.int32)), "U differs"
        # without U: the library's scratch holds it
        Y2 = torch.empty_like(Y)
        q.qlora_linear_fwd_noalloc(packed, codes, consts, X, A, B, alpha, Y2)
        torch.cuda.synchronize()
        assert torch.equal(Y2.view(torch.int16), Y_ref.view(torch.int16)), "Y differs without U_out"


def test_noalloc_forward_refuses_calls_beyond_its_scratch():
    import torch
    import nf4_bit_quantized_amd as q
    say("noalloc fwd beyond the static scratch")
    T, r, d_in, d_out = 40000, 64, 64, 64                  # needs 40000 * 512 bytes > 16 MiB
    assert q.qlora_fwd_workspace_bytes(d_out, d_in, T, r) > q.QLORA_STATIC_SCRATCH_BYTES
    packed, codes, consts, _, A, B = _layer(d_out, d_in, 1, r, seed=3)
    X = torch.zeros((T, d_in), dtype=torch.bfloat16, device="cuda")
    Y = torch.full((T, d_out), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(q.QloraError) as e:
        q.qlora_linear_fwd_noalloc(packed, codes, consts, X, A, B, 16.0, Y)
    assert e.value.status == q.QLORA_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert bool((Y == 7.0).all()), "a refused call wrote its output"
