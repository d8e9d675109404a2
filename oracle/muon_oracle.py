"""Plain fp64 CPU oracle of the Muon optimizer step.

TEST INFRASTRUCTURE ONLY.  This module is the yardstick the HIP library is
checked against.  Only the test suite, the smoke check and the CPU-baseline leg
of the benchmark may import it; the library's product path never does.  It
shares no code, constant table or helper with the HIP implementation, and it
never receives an expected value from it.

Everything is written as plainly as possible, in float64 numpy, following the
order of the steps on the pages.  Pages cited (their titles, sections and
snippets):

* [airosetta] "Muon optimizer: matrix-aware LLM optimizer" (airosetta.com,
  Cantonese), section "Muon's PyTorch implementation and core mechanism":
  the ``newtonschulz5`` routine and the ``Muon.step`` loop.
* [wmrh] "Muon meets Mamba" (wmrh.cn), sections 2.1 (what Muon does), 2.2
  (Newton-Schulz and polar decomposition), 4.1-4.2 (the optimizer class,
  ``_step_muon``).
* [csdn] "AdamW vs Muon / DeepSeek-V4" (adg.csdn.net), sections "Muon's core
  mechanism", "1. Preprocessing: normalisation", "2. Newton-Schulz
  iteration", "3. DeepSeek-V4 hybrid schedule" and "3. Scaling and update".

Readings taken where the pages are silent or disagree are stated at each
function (momentum as an EMA/lerp, eps added to the norm, strict ">" for the
transpose rule, sqrt(max(1, rows/cols)) for the RMS scale, decoupled weight
decay).

Every function here is pinned by ``tests/test_oracle_pins.py`` against
closed forms, invariants and textbook routines (numpy's SVD), not against
itself; ``tests/test_oracle_vs_torch_muon.py`` checks the whole step against
PyTorch's own ``torch.optim.Muon`` on the CPU.
"""
from __future__ import annotations

import numpy as np

# Quintic coefficients (a, b, c) printed in [airosetta]'s newtonschulz5 routine
# and in [csdn] section "3. DeepSeek-V4 hybrid schedule" (which misprints a as
# 3.445; the airosetta value is taken).
QUINTIC = (3.4445, -4.7750, 2.0315)
# Cubic Newton-Schulz X <- 1.5 X - 0.5 X X^T X of [wmrh] section 2.2, written
# as a (a, b, c) triple of the same polynomial family (c = 0).
CUBIC = (1.5, -0.5, 0.0)
# The gentle second stage of [csdn]'s hybrid schedule: (a, b, c) = (2, -1.5, 0.5).
HYBRID_TAIL = (2.0, -1.5, 0.5)

DEFAULT_EPS = 1e-7  # [airosetta] newtonschulz5 default eps


def as_f64(x) -> np.ndarray:
    """Upcast whatever exact values the caller holds (bf16 already widened
    to float32, or float32) to float64 without changing them."""
    return np.asarray(x, dtype=np.float64)


def momentum_lerp(m_prev, g, mu):
    """Momentum accumulation, EMA form:  M <- mu * M + (1 - mu) * G.

    [airosetta] Muon.step multiplies the buffer by the momentum and adds the
    gradient weighted by one minus the momentum; [wmrh] section 4.2
    ``_step_muon`` does the same.  ([csdn] writes the undamped sum
    M = mu M + G; with a zero initial buffer the two differ only by the
    constant factor (1 - mu), which the normalisation below removes.)
    """
    return mu * as_f64(m_prev) + (1.0 - mu) * as_f64(g)


def frobenius_norm(m) -> float:
    """||M||_F = sqrt(sum of squares), summed exactly enough in float64.

    [csdn] section "1. Preprocessing": the Frobenius norm is the square root of
    the sum of all squared entries.
    """
    m = as_f64(m)
    return float(np.sqrt(np.sum(m * m)))


def normalise(m, eps=DEFAULT_EPS):
    """X0 = M / (||M||_F + eps).

    [airosetta] newtonschulz5 divides by (norm + eps) with eps = 1e-7;
    [csdn] section "1. Preprocessing" explains that dividing by the Frobenius
    norm bounds the largest singular value by one.  eps is added to the norm,
    not to its square.
    """
    m = as_f64(m)
    return m / (frobenius_norm(m) + eps)


def needs_transpose(rows: int, cols: int) -> bool:
    """Work on the short side: transpose when rows > cols (strict, so square
    matrices are not transposed).  [airosetta] newtonschulz5; [wmrh] 2.2."""
    return rows > cols


def ns_iteration(x, a, b, c):
    """One quintic Newton-Schulz iteration on a wide (m <= n) matrix X:

        A = X X^T ;  B = b A + c A A ;  X' = a X + B X

    This is [airosetta]'s loop body, which [csdn] section "2. Newton-Schulz
    iteration" writes in expanded form a M + b (M M^T) M + c (M M^T)^2 M.
    """
    A = x @ x.T
    B = b * A + c * (A @ A)
    return a * x + B @ x


def newton_schulz(g, coeffs=(QUINTIC,), steps=5, eps=DEFAULT_EPS):
    """Orthogonalise G by `steps` Newton-Schulz iterations ([airosetta]
    newtonschulz5):  normalise by the Frobenius norm, transpose to the short
    side, iterate, transpose back.

    ``coeffs`` is either one (a, b, c) triple used for every step or one triple
    per step (for [csdn]'s hybrid schedule).
    """
    g = as_f64(g)
    if g.ndim != 2:
        raise ValueError("Newton-Schulz works on 2-D matrices only")
    coeffs = list(coeffs)
    if len(coeffs) == 1:
        coeffs = coeffs * steps
    if len(coeffs) != steps:
        raise ValueError("need one coefficient triple or one per step")
    x = normalise(g, eps)
    transposed = needs_transpose(*g.shape)
    if transposed:
        x = x.T
    for a, b, c in coeffs:
        x = ns_iteration(x, a, b, c)
    if transposed:
        x = x.T
    return x


def rms_scale(rows: int, cols: int, mode: str | None) -> float:
    """Per-matrix update scale.

    [csdn] section "3. Scaling and update" says the orthogonalised update has
    its RMS rescaled according to the matrix size but gives no formula.  The
    reading taken: s = sqrt(max(1, rows / cols)) on the stored rows x cols
    shape when the mode "sqrt_max1" is requested, else s = 1.
    """
    if mode is None or mode == "none":
        return 1.0
    if mode == "sqrt_max1":
        return float(np.sqrt(max(1.0, rows / cols)))
    raise ValueError(f"unknown rms scale mode {mode!r}")


def apply_update(p, o, lr, wd, scale):
    """Decoupled weight decay and update, both terms from the old parameter:

        p <- p * (1 - lr * wd) - lr * s * O

    [wmrh] section 4.2 ``_step_muon`` multiplies p by (1 - lr wd) before adding
    the orthogonalised step times -lr; [csdn] section "3. Scaling and update"
    applies standard weight decay and subtracts the scaled matrix.
    """
    return as_f64(p) * (1.0 - lr * wd) - lr * scale * as_f64(o)


def zero_center(g):
    """Subtract each column's mean: g - g.mean(dim=0, keepdim=True), the
    ``zerocenter`` helper of [wmrh] section 2.1 (applied by ``_step_muon`` in
    section 4.2 before the momentum).  Taken on the stored rows x cols
    gradient, before any transpose to the short side."""
    g = as_f64(g)
    return g - g.mean(axis=0, keepdims=True)


def nesterov_input(m_new, g, mu):
    """NS input of the look-ahead variant.  The pages carry a ``nesterov``
    flag but never define what it does ([wmrh] 4.1 accepts and ignores it;
    [airosetta] selects the buffer).  The reading taken for the variant: the
    iteration runs on mu * M_t + (1 - mu) * G_t, the gradient pulled toward
    the new momentum (with M_t itself the EMA of the gradients)."""
    return mu * as_f64(m_new) + (1.0 - mu) * as_f64(g)


def muon_step_matrix(p, g, m, *, lr=0.02, mu=0.95, wd=0.0, ns_steps=5,
                     coeffs=(QUINTIC,), eps=DEFAULT_EPS, rms_mode=None,
                     zero_centering=False, nesterov=False, ns_first=False):
    """One Muon step on one 2-D parameter, in the pages' order
    (momentum, then orthogonalisation, then decayed update; [wmrh] 4.2 picks
    momentum before Newton-Schulz, as does [airosetta]).

    Variants ([wmrh] sections 2.1 and 4.2):
    ``zero_centering`` subtracts the gradient's column means first;
    ``ns_first`` takes the other order the page discusses, zero-center ->
    Newton-Schulz -> momentum buffer -> update: the momentum averages the
    orthogonalised gradients and the update is -lr * s * M;
    ``nesterov`` runs the iteration on ``nesterov_input`` (not with
    ``ns_first``: the pages give that combination no meaning).

    Returns a dict with every stage so each can be compared on its own:
    ``m`` (new momentum), ``nu`` (Frobenius norm of the NS input), ``o``
    (orthogonalised matrix), ``p`` (new parameter), ``scale`` (the RMS scale
    used).  When ``g`` is None the matrix is skipped ([airosetta] Muon.step
    skips parameters without a gradient): nothing changes.
    """
    if g is None:
        return {"m": as_f64(m), "nu": None, "o": None, "p": as_f64(p), "scale": None}
    if nesterov and ns_first:
        raise ValueError("nesterov and ns_first together are not defined")
    rows, cols = np.shape(g)
    g = zero_center(g) if zero_centering else as_f64(g)
    s = rms_scale(rows, cols, rms_mode)
    if ns_first:
        nu = frobenius_norm(g)
        o = newton_schulz(g, coeffs, ns_steps, eps)
        m_new = momentum_lerp(m, o, mu)
        p_new = apply_update(p, m_new, lr, wd, s)
        return {"m": m_new, "nu": nu, "o": o, "p": p_new, "scale": s}
    m_new = momentum_lerp(m, g, mu)
    x = nesterov_input(m_new, g, mu) if nesterov else m_new
    nu = frobenius_norm(x)
    o = newton_schulz(x, coeffs, ns_steps, eps)
    p_new = apply_update(p, o, lr, wd, s)
    return {"m": m_new, "nu": nu, "o": o, "p": p_new, "scale": s}


def muon_step(params, grads, moms, **kw):
    """A list of matrices is simply the per-matrix step applied to each one
    (matrices are independent)."""
    return [muon_step_matrix(p, g, m, **kw) for p, g, m in zip(params, grads, moms)]

