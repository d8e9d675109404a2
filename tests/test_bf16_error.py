"""CPU pins of the first-order bf16 error estimate (tests/bf16_error.py).

The estimate is checked against what it claims to model, not against itself:
a Monte Carlo run of the fp64 iteration of "Muon optimizer: matrix-aware LLM"
(airosetta.com, newtonschulz5) with each documented rounding point replaced
by an explicit random relative perturbation of at most u = 2^-8 per entry
(uniform, symmetric matrices perturbed symmetrically).  The RMS relative
output error of those runs must agree with the estimate, over wide, tall,
square, very wide and unsplit-C shapes, so a dropped term or a wrong index
in the closed-form derivative shows up as a mismatch."""
import numpy as np
import pytest

from oracle import muon_oracle as O
from tests.bf16_error import U_BF16, ns_error_estimate, ns_error_estimate_for


def _perturb(z, rng, sym=False):
    r = rng.uniform(-1.0, 1.0, z.shape)
    if sym:
        r = np.triu(r)
        r = r + np.triu(r, 1).T
    return z * (1.0 + U_BF16 * r)


def _monte_carlo(g, coeffs, steps, split, trials, rng):
    x0 = np.asarray(g, np.float64) / np.linalg.norm(g)
    if x0.shape[0] > x0.shape[1]:
        x0 = x0.T
    ref = O.newton_schulz(x0, coeffs, steps, eps=0.0)
    acc = 0.0
    for _ in range(trials):
        x = _perturb(x0, rng)
        for k in range(steps):
            a, b, c = coeffs[0] if len(coeffs) == 1 else coeffs[k]
            A = _perturb(x @ x.T, rng, sym=True)
            C = a * np.eye(len(A)) + b * A + c * (A @ A)
            if not split:
                C = _perturb(C, rng, sym=True)
            x = _perturb(C @ x, rng)
        acc += np.linalg.norm(x - ref) ** 2
    return np.sqrt(acc / trials) / np.linalg.norm(ref)


@pytest.mark.parametrize("shape,split", [((20, 20), True), ((12, 30), False), ((3, 40), True),
                                         ((30, 12), True), ((16, 48), True)])
def test_estimate_matches_monte_carlo(shape, split):
    rng = np.random.default_rng(sum(shape))
    g = rng.standard_normal(shape)
    xs = np.linalg.svd(g / np.linalg.norm(g), compute_uv=False)
    est = ns_error_estimate(xs, *shape, (O.QUINTIC,), 5, c_split=split)
    mc = _monte_carlo(g, (O.QUINTIC,), 5, split, 200, rng)
    assert 0.75 <= mc / est <= 1.33, (shape, est, mc)


def test_estimate_matches_monte_carlo_square_small_pair():
    """A square matrix with two equal small singular values: the skew part of
    that pair is amplified by F(y) / y (the sum divided difference), which a
    random Gaussian matrix barely exercises."""
    rng = np.random.default_rng(11)
    u, _ = np.linalg.qr(rng.standard_normal((8, 8)))
    v, _ = np.linalg.qr(rng.standard_normal((8, 8)))
    s = np.array([1.0, 0.9, 0.8, 0.7, 0.6, 0.5, 0.05, 0.05])
    g = u @ np.diag(s) @ v.T
    xs = np.linalg.svd(g / np.linalg.norm(g), compute_uv=False)
    est = ns_error_estimate(xs, 8, 8, (O.QUINTIC,), 5)
    mc = _monte_carlo(g, (O.QUINTIC,), 5, True, 300, rng)
    assert 0.75 <= mc / est <= 1.33, (est, mc)


def test_estimate_matches_monte_carlo_hybrid_schedule():
    """Per-step coefficients: the 8 + 2 schedule of 'AdamW vs Muon'
    (adg.csdn.net, section 3, DeepSeek-V4 hybrid schedule)."""
    coeffs = [O.QUINTIC] * 8 + [O.HYBRID_TAIL] * 2
    rng = np.random.default_rng(7)
    g = rng.standard_normal((10, 24))
    xs = np.linalg.svd(g / np.linalg.norm(g), compute_uv=False)
    est = ns_error_estimate(xs, 10, 24, coeffs, 10)
    mc = _monte_carlo(g, coeffs, 10, True, 200, rng)
    assert 0.75 <= mc / est <= 1.33, (est, mc)


def test_estimate_special_cases():
    """The estimate is invariant under transposition and under scaling of the
    input; a zero matrix has no error; an exactly rank-one matrix does not
    survive bf16: the rounding noise in its null directions has singular
    values near u, which five quintic steps multiply by about a^5 = 486 (the
    slope of the map at 0), so the estimate is of order one."""
    rng = np.random.default_rng(1)
    g = rng.standard_normal((7, 11))
    e = ns_error_estimate_for(g, (O.QUINTIC,), 5)
    assert e == pytest.approx(ns_error_estimate_for(g.T, (O.QUINTIC,), 5), rel=1e-9)
    assert e == pytest.approx(ns_error_estimate_for(1e3 * g, (O.QUINTIC,), 5), rel=1e-6)
    u = rng.standard_normal((7, 1))
    v = rng.standard_normal((1, 11))
    r1 = ns_error_estimate_for(u @ v, (O.QUINTIC,), 5)
    assert r1 > 0.3
    assert ns_error_estimate(np.zeros(4), 4, 9, (O.QUINTIC,), 5) == 0.0


def test_estimate_grows_where_the_map_is_steep():
    """A normalised singular value near 2e-3 sits where five quintic steps
    amplify a perturbation about 480-fold: the estimate must say so."""
    u, _ = np.linalg.qr(np.random.default_rng(2).standard_normal((4, 4)))
    v, _ = np.linalg.qr(np.random.default_rng(3).standard_normal((6, 6)))
    well = np.array([0.6, 0.5, 0.45, 0.4])
    steep = np.array([0.6, 0.5, 0.45, 2e-3])
    def est(s):
        g = u @ np.diag(s) @ v[:4]
        return ns_error_estimate_for(g, (O.QUINTIC,), 5)
    assert est(steep) > 5 * est(well)
