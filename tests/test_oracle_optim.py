"""Pins of oracle.optim.adamw_step against things other than itself."""

import numpy as np
import pytest

from oracle import optim


def _torch_adamw(p0, grads, lr, betas, eps, wd):
    """torch.optim.AdamW on the CPU in float64: an independent implementation."""
    import torch
    p = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([p], lr=lr, betas=betas, eps=eps, weight_decay=wd, foreach=False)
    out = []
    for g in grads:
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        st = opt.state[p]
        out.append((p.detach().numpy().copy(), st["exp_avg"].numpy().copy(), st["exp_avg_sq"].numpy().copy()))
    return out


@pytest.mark.parametrize("lr,betas,eps,wd", [(1e-3, (0.9, 0.999), 1e-8, 0.01), (2e-4, (0.8, 0.95), 1e-6, 0.0),
                                             (5e-2, (0.5, 0.9), 1e-3, 0.1)])
def test_matches_torch_adamw(lr, betas, eps, wd):
    rng = np.random.default_rng(0)
    p0 = rng.standard_normal(257)
    grads = [rng.standard_normal(257) * 10.0 ** rng.uniform(-3, 1) for _ in range(6)]
    ref = _torch_adamw(p0, grads, lr, betas, eps, wd)
    p, m, v = p0, np.zeros_like(p0), np.zeros_like(p0)
    for t, (g, (pt, mt, vt)) in enumerate(zip(grads, ref), start=1):
        p, m, v = optim.adamw_step(p, g, m, v, t, lr, betas[0], betas[1], eps, wd)
        # torch forms m by linear interpolation (other rounding where the two
        # terms cancel): compare against the array's scale
        np.testing.assert_allclose(m, mt, rtol=1e-12, atol=1e-14 * np.max(np.abs(mt)))
        np.testing.assert_allclose(v, vt, rtol=1e-12, atol=1e-14 * np.max(np.abs(vt)))
        np.testing.assert_allclose(p, pt, rtol=1e-12, atol=1e-14 * np.max(np.abs(pt)))


def test_first_step_closed_form():
    # zero moments: m_hat = g, v_hat = g^2, so p moves by lr * g / (|g| + eps) after the decay
    g = np.array([3.0, -0.5, 1e-9, 0.0, -7.0])
    p0 = np.array([1.0, -2.0, 0.5, 4.0, 0.0])
    lr, eps, wd = 0.1, 1e-8, 0.2
    p, m, v = optim.adamw_step(p0, g, np.zeros(5), np.zeros(5), 1, lr, 0.9, 0.999, eps, wd)
    want = p0 * (1 - lr * wd) - lr * g / (np.abs(g) + eps)
    np.testing.assert_allclose(p, want, rtol=1e-14, atol=1e-17)
    np.testing.assert_allclose(m, 0.1 * g, rtol=1e-15)
    np.testing.assert_allclose(v, 0.001 * g * g, rtol=1e-15)


def test_decay_alone():
    p = np.array([2.0, -1.0])
    m = v = np.zeros(2)
    for t in range(1, 4):
        p, m, v = optim.adamw_step(p, np.zeros(2), m, v, t, 0.5, 0.9, 0.999, 1e-8, 0.1)
    np.testing.assert_allclose(p, np.array([2.0, -1.0]) * 0.95 ** 3, rtol=1e-15)


def test_grad_scale_is_a_gradient_multiplier():
    rng = np.random.default_rng(1)
    p0, g = rng.standard_normal(64), rng.standard_normal(64)
    z = np.zeros(64)
    a = optim.adamw_step(p0, g, z, z, 3, 1e-3, 0.9, 0.99, 1e-8, 0.01, grad_scale=0.25)
    b = optim.adamw_step(p0, g * 0.25, z, z, 3, 1e-3, 0.9, 0.99, 1e-8, 0.01)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def _planted(kind):
    def step(p, g, m, v, t, lr, b1, b2, eps, wd):
        p = np.array(p, np.float64)
        if kind == "coupled":          # L2 decay folded into the gradient (Adam, not AdamW)
            g = g + wd * p
        else:
            p = p * (1 - lr * wd)
        m = b1 * m + (1 - b1) * g
        v = b2 * v + (1 - b2) * g * g
        if kind == "no_bias_correction":
            return p - lr * m / (np.sqrt(v) + eps), m, v
        return p - lr * (m / (1 - b1 ** t)) / (np.sqrt(v / (1 - b2 ** t)) + eps), m, v
    return step


@pytest.mark.parametrize("kind", ["coupled", "no_bias_correction"])
def test_planted_mistakes_fail_the_torch_pin(kind):
    rng = np.random.default_rng(2)
    p0 = rng.standard_normal(33)
    grads = [rng.standard_normal(33) for _ in range(3)]
    ref = _torch_adamw(p0, grads, 1e-2, (0.9, 0.999), 1e-8, 0.05)
    bad = _planted(kind)
    p, m, v = p0, np.zeros(33), np.zeros(33)
    for t, g in enumerate(grads, start=1):
        p, m, v = bad(p, g, m, v, t, 1e-2, 0.9, 0.999, 1e-8, 0.05)
    assert not np.allclose(p, ref[-1][0], rtol=1e-10, atol=0)
