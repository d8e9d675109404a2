"""Pins of the fp64 AdamW oracle (``oracle.adamw_oracle``) to facts fixed by
the page's update rule ("Muon meets Mamba", section 4.2, ``_step_adamw``) and
by the mathematics, not to the oracle itself:

* first step from zero moments: the bias corrections make m_hat = g and
  v_hat = g^2 exactly, so the step is lr g / (|g| + eps);
* a constant gradient keeps m_hat = g, v_hat = g^2 at every step, so T steps
  move p by T lr g / (|g| + eps) (no decay);
* with eps = 0 the first step is lr sign(g), whatever the gradient's scale;
* a zero gradient only decays: p (1 - lr wd);
* the two-step moments equal their unrolled closed forms;
* a tensor without a gradient is left untouched.

Each check is run on the oracle and on deliberately broken copies of the
update (planted here, on the CPU): every copy must fail at least one check.
"""
import numpy as np
import pytest

import oracle

LR, B1, B2, EPS, WD = 1e-3, 0.9, 0.95, 1e-8, 0.01


def _rng(seed):
    return np.random.default_rng(seed)


def _check_first_step(step):
    r = _rng(1)
    p, g = r.normal(size=200), r.normal(size=200) * 3
    z = np.zeros(200)
    pn, m, v = step(p, g, z, z, 1, lr=LR, betas=(B1, B2), eps=EPS, wd=WD)
    want = p * (1 - LR * WD) - LR * g / (np.abs(g) + EPS)
    assert np.allclose(pn, want, rtol=0, atol=1e-15)
    assert np.allclose(m, (1 - B1) * g, rtol=1e-15) and np.allclose(v, (1 - B2) * g * g, rtol=1e-15)


def _check_constant_gradient(step):
    r = _rng(2)
    p0, g = r.normal(size=50), r.normal(size=50)
    p, m, v = p0.copy(), np.zeros(50), np.zeros(50)
    T = 25
    for t in range(1, T + 1):
        p, m, v = step(p, g, m, v, t, lr=LR, betas=(B1, B2), eps=EPS, wd=0.0)
    want = p0 - T * LR * g / (np.abs(g) + EPS)
    assert np.allclose(p, want, rtol=0, atol=1e-13)


def _check_scale_free(step):
    r = _rng(3)
    p, g = r.normal(size=64), r.normal(size=64)
    z = np.zeros(64)
    for k in (1e-6, 1.0, 1e6):
        pn, _, _ = step(p, k * g, z, z, 1, lr=LR, betas=(B1, B2), eps=0.0, wd=0.0)
        assert np.allclose(pn, p - LR * np.sign(g), rtol=0, atol=1e-15)


def _check_zero_gradient_decays(step):
    r = _rng(4)
    p = r.normal(size=32)
    m = np.zeros(32)
    pn, mn, vn = step(p, np.zeros(32), m, m, 3, lr=LR, betas=(B1, B2), eps=EPS, wd=WD)
    assert np.array_equal(pn, p * (1 - LR * WD)) and not mn.any() and not vn.any()


def _check_two_steps_closed_form(step):
    r = _rng(5)
    p, g1, g2 = r.normal(size=40), r.normal(size=40), r.normal(size=40)
    z = np.zeros(40)
    p1, m1, v1 = step(p, g1, z, z, 1, lr=LR, betas=(B1, B2), eps=EPS, wd=WD)
    p2, m2, v2 = step(p1, g2, m1, v1, 2, lr=LR, betas=(B1, B2), eps=EPS, wd=WD)
    m_want = B1 * (1 - B1) * g1 + (1 - B1) * g2
    v_want = B2 * (1 - B2) * g1 ** 2 + (1 - B2) * g2 ** 2
    assert np.allclose(m2, m_want, rtol=1e-14) and np.allclose(v2, v_want, rtol=1e-14)
    # bias corrections at t = 2: 1 - B^2
    upd = (LR / (1 - B1 ** 2)) * m_want / (np.sqrt(v_want / (1 - B2 ** 2)) + EPS)
    assert np.allclose(p2, p1 * (1 - LR * WD) - upd, rtol=0, atol=1e-15)


CHECKS = [_check_first_step, _check_constant_gradient, _check_scale_free,
          _check_zero_gradient_decays, _check_two_steps_closed_form]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__[7:])
def test_oracle_passes(check):
    check(oracle.adamw_step_tensor)


def test_missing_gradient_skips_the_tensor():
    p, m, v = np.ones(3), np.full(3, 0.5), np.full(3, 0.25)
    (pn, mn, vn), = oracle.adamw_step([p], [None], [m], [v], [7])
    assert np.array_equal(pn, p) and np.array_equal(mn, m) and np.array_equal(vn, v)
    with pytest.raises(ValueError):
        oracle.adamw_step_tensor(p, p, m, v, 0)


def _mutant(kind):
    def step(p, g, m, v, t, *, lr, betas, eps, wd):
        p, g, m, v = (np.asarray(x, dtype=np.float64) for x in (p, g, m, v))
        b1, b2 = betas
        if kind == "swapped_betas":
            b1, b2 = b2, b1
        if wd != 0 and kind != "decay_after":
            p = p * (1 - lr * wd)
        m = b1 * m + (1 - b1) * g
        v = b2 * v + (1 - b2) * (g if kind == "v_not_squared" else g * g)
        c1 = 1 - b1 ** t if kind != "no_bias_correction" else 1.0
        c2 = 1 - b2 ** t if kind != "no_bias_correction" else 1.0
        if kind == "eps_inside_sqrt":
            denom = np.sqrt(v / c2 + eps)
        elif kind == "c2_not_rooted":
            denom = np.sqrt(v) / c2 + eps
        else:
            denom = np.sqrt(v) / np.sqrt(c2) + eps
        pn = p - (lr / c1) * m / denom
        if wd != 0 and kind == "decay_after":
            pn = pn * (1 - lr * wd)
        if kind == "coupled_decay":
            pn = pn - lr * wd * pn
        return pn, m, v
    return step


@pytest.mark.parametrize("kind", ["swapped_betas", "no_bias_correction", "eps_inside_sqrt",
                                  "c2_not_rooted", "v_not_squared", "decay_after"])
def test_every_planted_mistake_fails_a_check(kind):
    failed = 0
    for check in CHECKS:
        try:
            check(_mutant(kind))
        except AssertionError:
            failed += 1
    assert failed >= 1, kind
