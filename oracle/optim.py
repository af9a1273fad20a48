"""AdamW update of the adapter parameters -- CPU oracle (float64).

TEST INFRASTRUCTURE ONLY (see ``oracle``): never imported by the product path.

What it follows: after the backward pass only the adapter matrices A and B
are updated by the optimizer, the quantized base weight never
([QLoRA-入门到精通] §3(3), an AdamW-type optimizer named there).  The pages do
not restate the optimizer's arithmetic; it is the published AdamW method
(Loshchilov and Hutter, "Decoupled Weight Decay Regularization"), in the form
in which the decay is applied to the parameter directly, scaled by the
learning rate, and the moment estimates are bias-corrected.  For step t >= 1
and gradient g (first multiplied by ``grad_scale``, e.g. 1 / the number of
accumulated micro-batches):

    p <- p * (1 - lr * weight_decay)
    m <- beta1 * m + (1 - beta1) * g
    v <- beta2 * v + (1 - beta2) * g^2
    p <- p - lr * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)

The paged placement of the optimizer state (moving it to host memory under
memory pressure) is not part of the arithmetic and is not modelled.

All arithmetic is float64.  Pins (``tests/test_oracle_optim.py``): several
steps against ``torch.optim.AdamW`` run on the CPU in float64 (an independent
implementation of the same method); the closed form of the first step from
zero moments (p moves by lr * g / (|g| + eps) after the decay); weight decay
alone (g = 0) scales p by (1 - lr * wd) per step; and planted mistakes
(bias correction dropped, decay applied to the gradient instead) fail them.
"""

import numpy as np


def adamw_step(p, g, m, v, step: int, lr: float, beta1: float, beta2: float, eps: float,
               weight_decay: float, grad_scale: float = 1.0):
    """One AdamW step; returns new (p, m, v) as float64 arrays (inputs untouched)."""
    assert step >= 1
    p = np.array(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64) * grad_scale
    m = np.array(m, dtype=np.float64)
    v = np.array(v, dtype=np.float64)
    # decoupled weight decay: on the parameter, scaled by the learning rate
    p = p * (1.0 - lr * weight_decay)
    # moment estimates
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    # bias-corrected update
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v
