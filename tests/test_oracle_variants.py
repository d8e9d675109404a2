"""Pins of the oracle's variant options ("Muon meets Mamba", sections 2.1 and
4.2: zero-centering, and the Newton-Schulz-then-momentum order; and the
look-ahead reading of the "nesterov" flag) against facts independent of the
oracle's own code: hand-computed means, column-constant gradients, the
scale invariance of the iteration, and numpy's SVD polar factor reached by
the cubic iteration.  Planted mistakes in CPU copies of the variant code must
each fail a check."""
import numpy as np
import pytest

import oracle

CUBIC30 = dict(coeffs=(oracle.CUBIC,), ns_steps=30, eps=0.0)


def _polar(g):
    u, _, vt = np.linalg.svd(np.asarray(g, np.float64), full_matrices=False)
    return u @ vt


def _well_conditioned(r, c, seed):
    rng = np.random.default_rng(seed)
    u, _ = np.linalg.qr(rng.standard_normal((r, min(r, c))))
    v, _ = np.linalg.qr(rng.standard_normal((c, min(r, c))))
    s = np.linspace(1.0, 0.3, min(r, c))
    return (u * s) @ v.T


def check_zero_center_by_hand(step):
    g = np.array([[1.0, 2.0, 3.0], [3.0, 4.0, 5.0]])
    want = np.array([[-1.0, -1.0, -1.0], [1.0, 1.0, 1.0]])
    out = step(np.zeros((2, 3)), g, np.zeros((2, 3)), lr=1.0, mu=0.0, wd=0.0, ns_steps=0,
               zero_centering=True)
    assert np.allclose(out["m"], want, atol=1e-15)


def check_column_constant_gradient_gives_no_update(step):
    rng = np.random.default_rng(1)
    # every row the same, values on a 1/8 grid so the column means are exact
    g = np.ones((12, 1)) * (np.round(rng.normal(size=(1, 20)) * 8) / 8)
    p = rng.normal(size=(12, 20))
    out = step(p, g, np.zeros((12, 20)), lr=0.02, mu=0.95, wd=0.01, zero_centering=True)
    assert np.abs(out["o"]).max() == 0.0
    assert np.array_equal(out["p"], p * (1 - 0.02 * 0.01))


def check_centered_columns_have_zero_mean(step):
    rng = np.random.default_rng(2)
    g = rng.normal(size=(9, 5)) + 3.0
    out = step(np.zeros((9, 5)), g, np.zeros((9, 5)), lr=1.0, mu=0.0, wd=0.0, ns_steps=0,
               zero_centering=True)
    assert np.abs(out["m"].sum(axis=0)).max() < 1e-13
    assert np.abs(out["m"].sum(axis=1)).max() > 1e-3      # rows are not centered


def check_nesterov_first_step_equals_plain(step):
    rng = np.random.default_rng(3)
    g = rng.normal(size=(16, 40))
    a = step(np.zeros((16, 40)), g, np.zeros((16, 40)), eps=0.0)
    b = step(np.zeros((16, 40)), g, np.zeros((16, 40)), eps=0.0, nesterov=True)
    assert np.allclose(a["o"], b["o"], rtol=0, atol=1e-12)


def check_nesterov_second_step_polar(step):
    mu = 0.9
    g1, g2 = _well_conditioned(8, 14, 4), _well_conditioned(8, 14, 5)
    s1 = step(np.zeros((8, 14)), g1, np.zeros((8, 14)), mu=mu, nesterov=True, **CUBIC30)
    s2 = step(np.zeros((8, 14)), g2, s1["m"], mu=mu, nesterov=True, **CUBIC30)
    want = _polar(mu * mu * s1["m"] + (1 - mu * mu) * g2)
    assert np.allclose(s2["o"], want, atol=1e-9)


def check_ns_first_polar(step):
    mu, lr, wd = 0.9, 0.1, 0.01
    g1, g2 = _well_conditioned(10, 6, 6), _well_conditioned(10, 6, 7)
    p0 = np.random.default_rng(8).normal(size=(10, 6))
    s1 = step(p0, g1, np.zeros((10, 6)), mu=mu, lr=lr, wd=wd, ns_first=True, **CUBIC30)
    assert np.allclose(s1["m"], (1 - mu) * _polar(g1), atol=1e-9)
    assert np.allclose(s1["p"], p0 * (1 - lr * wd) - lr * (1 - mu) * _polar(g1), atol=1e-9)
    s2 = step(s1["p"], g2, s1["m"], mu=mu, lr=lr, wd=wd, ns_first=True, **CUBIC30)
    assert np.allclose(s2["m"], mu * (1 - mu) * _polar(g1) + (1 - mu) * _polar(g2), atol=1e-9)


def check_centered_ns_first(step):
    g = _well_conditioned(7, 11, 9) + 0.5
    out = step(np.zeros((7, 11)), g, np.zeros((7, 11)), mu=0.0, ns_first=True, zero_centering=True,
               **CUBIC30)
    c = g - g.mean(axis=0)
    # the centered matrix has rank <= 6 (its rows sum to zero): polar factor on its range
    u, s, vt = np.linalg.svd(c, full_matrices=False)
    k = int((s > 1e-8 * s[0]).sum())
    assert np.allclose(out["o"], u[:, :k] @ vt[:k], atol=1e-7)


CHECKS = [check_zero_center_by_hand, check_column_constant_gradient_gives_no_update,
          check_centered_columns_have_zero_mean, check_nesterov_first_step_equals_plain,
          check_nesterov_second_step_polar, check_ns_first_polar, check_centered_ns_first]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__[6:])
def test_oracle_passes(check):
    check(oracle.muon_step_matrix)


def test_nesterov_with_ns_first_is_rejected():
    with pytest.raises(ValueError):
        oracle.muon_step_matrix(np.zeros((2, 2)), np.ones((2, 2)), np.zeros((2, 2)), nesterov=True,
                                ns_first=True)


def _mutant(kind):
    def step(p, g, m, *, lr=0.02, mu=0.95, wd=0.0, ns_steps=5, coeffs=(oracle.QUINTIC,),
             eps=oracle.DEFAULT_EPS, rms_mode=None, zero_centering=False, nesterov=False, ns_first=False):
        g = np.asarray(g, np.float64)
        if zero_centering:
            g = g - (g.mean(axis=1, keepdims=True) if kind == "center_rows" else g.mean(axis=0, keepdims=True))
        if ns_first:
            o = oracle.newton_schulz(g, coeffs, ns_steps, eps)
            m_new = mu * np.asarray(m) + (1 - mu) * o
            upd = o if kind == "ns_first_updates_with_o" else m_new
            return {"m": m_new, "o": o, "p": np.asarray(p) * (1 - lr * wd) - lr * upd}
        m_new = mu * np.asarray(m) + (1 - mu) * g
        if nesterov:
            base = np.asarray(m) if kind == "nesterov_old_momentum" else m_new
            x = mu * base + (1 - mu) * g
        else:
            x = m_new
        o = oracle.newton_schulz(x, coeffs, ns_steps, eps)
        return {"m": m_new, "o": o, "p": np.asarray(p) * (1 - lr * wd) - lr * o}
    return step


@pytest.mark.parametrize("kind", ["center_rows", "ns_first_updates_with_o", "nesterov_old_momentum"])
def test_every_planted_mistake_fails_a_check(kind):
    failed = 0
    for check in CHECKS:
        try:
            check(_mutant(kind))
        except AssertionError:
            failed += 1
    assert failed >= 1, kind
