"""First-order estimate of the bf16 rounding error of the Newton-Schulz
output, computed from the fp64 oracle's spectrum of the normalised input.

The iteration is the newtonschulz5 routine of "Muon optimizer: matrix-aware
LLM" (airosetta.com): X0 = M / (||M||_F + eps), then per step A = X X^T,
B = b A + c A^2, X <- a X + B X, all on the short side.  The pages cast X to
bf16 and run every product in bf16; the library's documented rounding points
(include/muon.h) are: X0, A, C = a I + b A + c A^2 and each new X, each
rounded once to nearest-even bf16 (unit roundoff u = 2^-8), with C carried as
a hi/lo pair (error ~u^2, neglected) when the short side is at most 128.

Each rounding perturbs one intermediate by a matrix whose entries are bounded
by u times the entry itself; modelled as independent and uniform on that
interval (variance u^2 |z|^2 / 3), its effect on the output is the Frechet
derivative of the rest of the iteration applied to it.  The iteration maps
every singular value x of X0 through the scalar polynomial p(x) = a x + b x^3
+ c x^5 and keeps the singular vectors, so each derivative has a closed form
in the singular basis of the generalised matrix function X -> U F(S) V^T
(F = the remaining composition of p): gain F'(y_i) on the diagonal, the
divided differences (F(y_i) - F(y_j)) / (y_i - y_j) and
(F(y_i) + F(y_j)) / (y_i + y_j) on the symmetric and skew parts of each
off-diagonal pair, and F(y_i) / y_i on the n - m extra columns.  The estimate
is the root of the summed variances (every rounding point, in quadrature),
relative to ||O||_F.  It is an expected size, not a worst case: the observed
error of a correct bf16 iteration falls around 0.7 of it, and a sum of a few
tens of independent contributions stays below 4 times it.

Test code only: it uses the method's mathematics and the documented rounding
points, never the library or a model of its kernels.
"""
from __future__ import annotations

import numpy as np

U_BF16 = 2.0 ** -8          # unit roundoff of bf16 round-to-nearest (8-bit significand)


def _p(x, a, b, c):
    return a * x + b * x ** 3 + c * x ** 5


def _orbit(xs, coeffs, k0, k1):
    """Singular values after steps k0 .. k1-1 applied to xs."""
    y = np.array(xs, dtype=np.float64)
    for k in range(k0, k1):
        y = _p(y, *coeffs[k])
    return y


def _gains(y, coeffs, k0, k1):
    """F = steps k0 .. k1-1 composed: F(y), F'(y) and F(y)/y (F is odd)."""
    f = np.array(y, dtype=np.float64)
    d = np.ones_like(f)
    q = np.ones_like(f)
    for k in range(k0, k1):
        a, b, c = coeffs[k]
        d = d * (a + 3 * b * f ** 2 + 5 * c * f ** 4)
        q = q * (a + b * f ** 2 + c * f ** 4)
        f = _p(f, a, b, c)
    return f, d, q


def _divided(y, f, d):
    """(F(yi) - F(yj)) / (yi - yj) (F' at coincident values) and
    (F(yi) + F(yj)) / (yi + yj) for every pair."""
    yi, yj = y[:, None], y[None, :]
    fi, fj = f[:, None], f[None, :]
    dif, tot = yi - yj, yi + yj
    close = np.abs(dif) <= 1e-12 * np.maximum(np.abs(yi), 1e-300)
    dm = np.where(close, (d[:, None] + d[None, :]) / 2, (fi - fj) / np.where(close, 1.0, dif))
    dp = np.where(tot > 0, (fi + fj) / np.where(tot > 0, tot, 1.0), 0.0)
    return dm, dp


def ns_error_estimate(xs, rows: int, cols: int, coeffs, steps: int,
                      c_split: bool | None = None) -> float:
    """Expected relative Frobenius error of the bf16 iteration's output.

    xs: singular values of the normalised input X0 (any order), as the fp64
    oracle computes them; coeffs: one (a, b, c) or one per step; c_split: C
    carried as a hi/lo pair (default: short side <= 128)."""
    coeffs = list(coeffs)
    if len(coeffs) == 1:
        coeffs = coeffs * steps
    m, n = min(rows, cols), max(rows, cols)
    if c_split is None:
        c_split = m <= 128
    xs = np.zeros(m) if len(xs) == 0 else np.asarray(xs, np.float64)
    xs = np.concatenate([xs, np.zeros(m - len(xs))]) if len(xs) < m else xs[:m]
    u2 = U_BF16 * U_BF16 / 3.0
    iu = np.triu_indices(m, 1)
    var = 0.0
    for k in range(steps + 1):
        y = _orbit(xs, coeffs, 0, k)
        # rounding of X_k (X_steps is the output itself)
        f, d, q = _gains(y, coeffs, k, steps)
        dm, dp = _divided(y, f, d)
        hs = np.sum(d ** 2) + np.sum(dm[iu] ** 2 + dp[iu] ** 2) + (n - m) * np.sum(q ** 2)
        var += u2 * np.sum(y ** 2) / (m * n) * hs
        if k == steps:
            break
        a, b, c = coeffs[k]
        y2 = y ** 2
        z = _p(y, a, b, c)
        f, d, q = _gains(z, coeffs, k + 1, steps)
        dm, dp = _divided(z, f, d)
        yi, yj = y[:, None], y[None, :]
        # rounding of A_k (symmetric): dX' = (b dA + c (dA A + A dA)) X
        g = b + c * (y2[:, None] + y2[None, :])
        s_part, k_part = g * (yi + yj) / 2, g * (yj - yi) / 2
        tot = np.sum((d * np.diag(g) * y) ** 2) + np.sum(
            (2 * (dm ** 2 * s_part ** 2 + dp ** 2 * k_part ** 2))[iu])
        var += u2 * np.sum(y2 ** 2) / (m * m) * tot
        # rounding of C_k when it is a single bf16 matrix: dX' = dC X
        if not c_split:
            cc = a + b * y2 + c * y2 ** 2
            s_part, k_part = (yi + yj) / 2, (yj - yi) / 2
            tot = np.sum((d * y) ** 2) + np.sum(
                (2 * (dm ** 2 * s_part ** 2 + dp ** 2 * k_part ** 2))[iu])
            var += u2 * np.sum(cc ** 2) / (m * m) * tot
    out = np.linalg.norm(_orbit(xs, coeffs, 0, steps))
    return float(np.sqrt(var) / out) if out > 0 else 0.0


def ns_error_estimate_for(m_new, coeffs, steps: int, eps: float = 1e-7) -> float:
    """ns_error_estimate for the iteration run on momentum m_new (normalised
    by ||m_new||_F + eps, as the oracle does)."""
    m_new = np.asarray(m_new, np.float64)
    x = m_new / (np.linalg.norm(m_new) + eps)
    xs = np.linalg.svd(x, compute_uv=False)
    return ns_error_estimate(xs, *m_new.shape, coeffs, steps)
