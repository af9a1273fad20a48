"""Calls enqueue on the caller's stream (torch's current stream through the
binding): a layer step on a side stream gives the same bytes as on the
default stream, and waits for work queued before it on that stream."""

import numpy as np
import pytest

import workloads
from gpu_helpers import dev_bf16, dev_f32

pytestmark = pytest.mark.gpu


def _step(q, W, X, A, B, dY, alpha):
    import torch
    packed, codes, consts = q.qlora_quantize_nf4(W)
    Y, U = q.qlora_linear_fwd(packed, codes, consts, X, A, B, alpha)
    dX, dA, dB = q.qlora_linear_bwd(packed, codes, consts, X, A, B, alpha, dY, U_in=U)
    A32 = A.float()
    m, v = torch.zeros_like(A32), torch.zeros_like(A32)
    A16 = q.qlora_adamw_step(A32, dA, m, v, 1, 1e-3, weight_decay=0.01, param_bf16=A.clone())
    return [packed, codes, consts, Y, U, dX, dA, dB, A32, A16]


def test_side_stream_matches_default_stream():
    import nf4_bit_quantized_amd as q
    import torch
    inp = workloads.layer_inputs(256, 320, 48, 16, seed=170)
    W = dev_f32(inp["W"])
    X, A, B, dY = (dev_bf16(inp[k]) for k in ("X", "A", "B", "dY"))
    ref = _step(q, W, X, A, B, dY, 16.0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        # work queued first on the same stream: the layer's inputs are written there
        W2 = W * 1.0
        X2 = X.clone()
        got = _step(q, W2, X2, A, B, dY, 16.0)
    side.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                           b.view(torch.uint8) if b.dtype != torch.uint8 else b)
