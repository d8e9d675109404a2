"""Plain fp64 CPU oracle of the AdamW branch that accompanies Muon.

TEST INFRASTRUCTURE ONLY (same rules as ``oracle.muon_oracle``): imported by
the tests, the smoke check and the benchmark's CPU-baseline leg, never by the
library, and sharing no code with the HIP implementation.

Source: "Muon meets Mamba" (wmrh.cn), section 4.2, the ``_step_adamw`` method
of the optimizer class, with the defaults of its constructor in section 4.1
(AdamW learning rate 1e-3, betas (0.9, 0.95), eps 1e-8, weight decay shared
with the Muon group, 0.01).  Section 1.3 of the same page writes the moment
recursions as formulas.  Per parameter with a gradient, in the page's order:

1. decoupled decay with the AdamW learning rate: p <- p (1 - lr wd);
2. the step count t of this parameter goes up by one (t = 1 on the first call);
3. m <- beta1 m + (1 - beta1) g,  v <- beta2 v + (1 - beta2) g^2;
4. with the bias corrections c1 = 1 - beta1^t and c2 = 1 - beta2^t:
   p <- p - (lr / c1) * m / (sqrt(v) / sqrt(c2) + eps).

A parameter without a gradient is skipped entirely (no decay, no state change).
Every function is pinned by ``tests/test_oracle_adamw.py``.
"""
from __future__ import annotations

import numpy as np

ADAMW_LR = 1e-3
ADAMW_BETAS = (0.9, 0.95)
ADAMW_EPS = 1e-8
ADAMW_WD = 0.01


def adamw_step_tensor(p, g, m, v, t, *, lr=ADAMW_LR, betas=ADAMW_BETAS, eps=ADAMW_EPS,
                      wd=ADAMW_WD):
    """One AdamW update of one tensor.  ``t`` is this update's step count
    (already incremented, >= 1).  Returns (p_new, m_new, v_new) in float64;
    the inputs are upcast from the exact values the GPU sees."""
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    beta1, beta2 = betas
    if t < 1:
        raise ValueError("the step count of an update is >= 1")
    if wd != 0:
        p = p * (1.0 - lr * wd)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    c1 = 1.0 - beta1 ** t
    c2 = 1.0 - beta2 ** t
    denom = np.sqrt(v) / np.sqrt(c2) + eps
    p = p - (lr / c1) * m / denom
    return p, m, v


def adamw_step(params, grads, exp_avgs, exp_avg_sqs, steps, **kw):
    """List form: grads[i] is None skips tensor i (returned unchanged)."""
    out = []
    for p, g, m, v, t in zip(params, grads, exp_avgs, exp_avg_sqs, steps):
        if g is None:
            out.append((np.asarray(p, np.float64), np.asarray(m, np.float64),
                        np.asarray(v, np.float64)))
        else:
            out.append(adamw_step_tensor(p, g, m, v, t, **kw))
    return out
