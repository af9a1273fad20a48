"""GPU parity of the AdamW update of the adapter parameters against the
oracle (float64), over several steps from the same fp32 start, at sizes with
a ragged tail; the bf16 copy is the round-to-nearest-even of the fp32 result."""

import numpy as np
import pytest

from gpu_helpers import say
from oracle import optim
from oracle.bf16 import round_to_bf16

pytestmark = pytest.mark.gpu


def _state(n, seed):
    rng = np.random.default_rng(seed)
    p = (rng.standard_normal(n) * 0.05).astype(np.float32)
    grads = [(rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 0)).astype(np.float32) for _ in range(5)]
    return p, grads


@pytest.mark.parametrize("n", [1, 3, 5, 1024, 4097, (1 << 20) + 7])
@pytest.mark.parametrize("hp", [dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01, grad_scale=1.0),
                                dict(lr=2e-4, betas=(0.8, 0.95), eps=1e-6, weight_decay=0.0, grad_scale=0.25)])
def test_adamw_matches_oracle(n, hp):
    import nf4_bit_quantized_amd as q
    import torch
    say(f"adamw n={n} {hp}")
    p0, grads = _state(n, seed=n % 1000)
    P = torch.from_numpy(p0.copy()).cuda()
    M = torch.zeros(n, device="cuda")
    V = torch.zeros(n, device="cuda")
    P16 = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    p, m, v = p0.astype(np.float64), np.zeros(n), np.zeros(n)
    # the hyperparameters cross the C ABI as fp32: the oracle takes the same values
    f = lambda x: float(np.float32(x))
    hp32 = dict(lr=f(hp["lr"]), betas=(f(hp["betas"][0]), f(hp["betas"][1])), eps=f(hp["eps"]),
                weight_decay=f(hp["weight_decay"]), grad_scale=f(hp["grad_scale"]))
    for t, g in enumerate(grads, start=1):
        G = torch.from_numpy(g).cuda()
        q.qlora_adamw_step(P, G, M, V, t, hp["lr"], hp["betas"], hp["eps"], hp["weight_decay"], hp["grad_scale"],
                           param_bf16=P16)
        p, m, v = optim.adamw_step(p, g, m, v, t, hp32["lr"], hp32["betas"][0], hp32["betas"][1], hp32["eps"],
                                   hp32["weight_decay"], hp32["grad_scale"])
    torch.cuda.synchronize()
    gp, gm, gv = (x.cpu().numpy().astype(np.float64) for x in (P, M, V))
    # fp32 state after five steps: each step rounds p, m and v once or twice
    # (a few ulp of each) and the update term carries a relative error of a
    # few ulp, so 1e-6 of the largest value (about 8 ulp) bounds them all
    for got, want, nm in ((gp, p, "p"), (gm, m, "m"), (gv, v, "v")):
        err = np.max(np.abs(got - want)) / max(np.max(np.abs(want)), 1e-30)
        say(f"  {nm} {err:.2e}")
        assert err <= 1e-6, nm
    # the update itself, relative to its size (p - p0 is about lr per step)
    du_err = np.max(np.abs((gp - p0) - (p - p0))) / np.max(np.abs(p - p0))
    say(f"  update {du_err:.2e}")
    assert du_err <= 1e-3
    # bf16 copy: round-to-nearest-even of the kernel's own fp32 parameters
    got16 = P16.view(torch.int16).cpu().numpy().view(np.uint16)
    want16 = (round_to_bf16(P.cpu().numpy()).view(np.uint32) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(got16, want16)


def test_adamw_zero_size_is_a_no_op():
    import nf4_bit_quantized_amd as q
    import torch
    e = torch.empty(0, device="cuda")
    q.qlora_adamw_step(e, e, e, e, 1, 1e-3)
    torch.cuda.synchronize()
