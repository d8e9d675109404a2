"""Pins of the fp64 oracle against facts that do not come from the oracle
itself: closed forms, invariants, a textbook routine (numpy's SVD), exact
rational arithmetic and brute force on tiny inputs.

Each check is a function that takes the Newton-Schulz routine under test, so
the same checks can be run against deliberately broken copies of it
(``test_oracle_mutants.py``) to show that a plausible mistake fails at least
one of them.

Pages: [airosetta] newtonschulz5 / Muon.step; [wmrh] sections 2.2 and 4.2;
[csdn] sections on normalisation, the Newton-Schulz polynomial, the hybrid
schedule and the scaled update.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import muon_oracle as O

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "coefficients.json")))
QUINTIC = tuple(GOLDEN["quintic"]["value"])
CUBIC = tuple(GOLDEN["cubic"]["value"])


def rng(*k):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([900, *k])))


def rel(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


def haar(n, r):
    q, rr = np.linalg.qr(r.standard_normal((n, n)))
    return q * np.sign(np.diag(rr))


def scalar_map(x, coeffs, steps):
    """p_k(x) = a x + b x^3 + c x^5 applied `steps` times to a scalar / array:
    the action of the iteration on one singular value ([csdn] section
    "2. Newton-Schulz iteration": the matrix polynomial acts on singular values
    only)."""
    coeffs = list(coeffs)
    if len(coeffs) == 1:
        coeffs = coeffs * steps
    x = np.asarray(x, dtype=np.float64)
    for a, b, c in coeffs:
        x = a * x + b * x ** 3 + c * x ** 5
    return x


# ---------------------------------------------------------------------------
# reusable checks (take the NS routine under test)
# ---------------------------------------------------------------------------
def check_cubic_converges_to_polar(ns):
    """[wmrh] 2.2: the cubic iteration converges to the orthogonal polar
    factor; [csdn]: the target is U V^T from the SVD.  Wide and tall."""
    g = rng(1).standard_normal((64, 192))
    for mat in (g, g.T):
        u, s, vt = np.linalg.svd(mat, full_matrices=False)
        x = ns(mat, (CUBIC,), 30, 1e-7)
        assert rel(x, u @ vt) <= 1e-12


def check_transpose(ns):
    """NS(G^T) = NS(G)^T: the short-side rule only changes the work order."""
    g = rng(2).standard_normal((48, 80))
    assert rel(ns(g.T, (QUINTIC,), 5, 1e-7), ns(g, (QUINTIC,), 5, 1e-7).T) <= 1e-13
    s = rng(3).standard_normal((40, 40))
    assert rel(ns(s.T, (QUINTIC,), 5, 1e-7), ns(s, (QUINTIC,), 5, 1e-7).T) <= 1e-12


def check_scale_invariance(ns):
    """NS(cG) = NS(G) for c > 0 (exact with eps = 0; the eps term perturbs by
    about eps / (c ||G||))."""
    g = rng(4).standard_normal((32, 96))
    base = ns(g, (QUINTIC,), 5, 0.0)
    for c in (1e3, 1e-3, 7.0):
        assert rel(ns(c * g, (QUINTIC,), 5, 0.0), base) <= 1e-13
    nrm = np.linalg.norm(g)
    for c in (1e3, 1e-3):
        bound = 10 * 1e-7 / (c * nrm) + 1e-13
        assert rel(ns(c * g, (QUINTIC,), 5, 1e-7), ns(g, (QUINTIC,), 5, 0.0)) <= bound


def check_singular_value_map(ns, shape=(24, 40), steps=5, coeffs=(QUINTIC,)):
    """Closed form on G = U diag(s) V^T: the iteration keeps U and V and maps
    each normalised singular value through the scalar polynomial, so
    NS(G) = U diag(p^k(s / ||s||)) V^T ([csdn] section "2. Newton-Schulz
    iteration")."""
    m, n = shape
    r = rng(5, m, n)
    k = min(m, n)
    u = haar(m, r)[:, :k]
    v = haar(n, r)[:, :k]
    s = np.geomspace(1.0, 1e-2, k)
    g = (u * s) @ v.T
    want = (u * scalar_map(s / np.linalg.norm(s), coeffs, steps)) @ v.T
    assert rel(ns(g, coeffs, steps, 0.0), want) <= 1e-12


def check_orthogonal_equivariance(ns):
    """NS(P G Q^T) = P NS(G) Q^T for orthogonal P, Q."""
    r = rng(6)
    g = r.standard_normal((20, 36))
    p, q = haar(20, r), haar(36, r)
    assert rel(ns(p @ g @ q.T, (QUINTIC,), 5, 1e-7), p @ ns(g, (QUINTIC,), 5, 1e-7) @ q.T) <= 1e-12


def check_diagonal(ns):
    """A rectangular diagonal input stays diagonal, each entry mapped by the
    scalar polynomial."""
    d = np.array([3.0, 1.0, 0.5, 0.25, 0.01])
    for shape in ((5, 9), (9, 5)):
        g = np.zeros(shape)
        g[np.arange(5), np.arange(5)] = d
        want = np.zeros(shape)
        want[np.arange(5), np.arange(5)] = scalar_map(d / np.linalg.norm(d), (QUINTIC,), 5)
        assert np.max(np.abs(ns(g, (QUINTIC,), 5, 0.0) - want)) <= 1e-14


def check_rank_one(ns):
    """G = sigma u v^T gives X0 = u v^T and O = p^5(1) u v^T, where the orbit
    of 1 under p is computed in exact rational arithmetic from the printed
    coefficients."""
    a, b, c = (Fraction(str(x)) for x in QUINTIC)
    x = Fraction(1)
    orbit = []
    for _ in range(5):
        x = a * x + b * x ** 3 + c * x ** 5
        orbit.append(x)
    assert orbit[0] == Fraction(GOLDEN["quintic_at_one"]["value"])
    r = rng(7)
    u = r.standard_normal(16); u /= np.linalg.norm(u)
    v = r.standard_normal(28); v /= np.linalg.norm(v)
    for sigma in (1.0, 37.5):
        g = sigma * np.outer(u, v)
        got = ns(g, (QUINTIC,), 5, 0.0)
        assert rel(got, float(orbit[-1]) * np.outer(u, v)) <= 1e-13


def check_brute_force_tiny(ns):
    """One iteration on a 2 x 3 input, written out with explicit sums."""
    g = np.array([[1.0, -2.0, 0.5], [0.25, 3.0, -1.0]])
    nrm = math.sqrt(sum(v * v for v in g.ravel()))
    x = [[g[i][j] / nrm for j in range(3)] for i in range(2)]
    a, b, c = QUINTIC
    A = [[sum(x[i][k] * x[j][k] for k in range(3)) for j in range(2)] for i in range(2)]
    AA = [[sum(A[i][k] * A[k][j] for k in range(2)) for j in range(2)] for i in range(2)]
    B = [[b * A[i][j] + c * AA[i][j] for j in range(2)] for i in range(2)]
    want = np.array([[a * x[i][k] + sum(B[i][j] * x[j][k] for j in range(2)) for k in range(3)]
                     for i in range(2)])
    assert np.max(np.abs(ns(g, (QUINTIC,), 1, 0.0) - want)) <= 1e-14
    # tall input: the same numbers, transposed
    assert np.max(np.abs(ns(g.T, (QUINTIC,), 1, 0.0) - want.T)) <= 1e-14


ALL_CHECKS = [check_cubic_converges_to_polar, check_transpose, check_scale_invariance,
              check_singular_value_map, check_orthogonal_equivariance, check_diagonal,
              check_rank_one, check_brute_force_tiny]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_newton_schulz_pins(check):
    check(O.newton_schulz)


# ---------------------------------------------------------------------------
# band of the quintic, spectral bound, hybrid schedule
# ---------------------------------------------------------------------------
def test_quintic_band_and_spectral_bound():
    """The quintic does not converge to 1 (p(1) = 0.701) but pushes every
    normalised singular value >= 2e-3 into a band around 1 ([airosetta]:
    operator norm close to 1 after 5 steps).  The band is taken from the
    scalar map on a fine grid; the matrix oracle must land inside it for an
    input of condition number 1e4."""
    grid = np.geomspace(2e-3, 1.0, 200001)
    mapped = scalar_map(grid, (QUINTIC,), 5)
    lo, hi = mapped.min(), mapped.max()
    assert 0.68 < lo < 0.69 and 1.20 < hi < 1.21
    r = rng(8)
    m, n = 30, 50
    u, v = haar(m, r), haar(n, r)[:, :m]
    s = np.geomspace(1.0, 1e-4, m)
    s = s / np.linalg.norm(s)
    s = np.maximum(s, 2e-3)           # keep every normalised value >= 2e-3
    g = (u * s) @ v.T
    sv = np.linalg.svd(O.newton_schulz(g, (QUINTIC,), 5, 0.0), compute_uv=False)
    assert sv.min() >= lo - 1e-12 and sv.max() <= hi + 1e-12
    # spectral bound for any input: max of p^5 over [0, 1]
    full = scalar_map(np.linspace(0.0, 1.0, 200001), (QUINTIC,), 5).max()
    for seed in range(4):
        g = rng(9, seed).standard_normal((40, 64)) * rng(10, seed).standard_t(2, (40, 64))
        assert np.linalg.norm(O.newton_schulz(g), 2) <= full + 1e-12


def test_hybrid_schedule_locks_to_one():
    """[csdn] hybrid schedule: 8 quintic + 2 (2, -1.5, 0.5) steps.  q(1) = 1
    and q'(1) = 0, so singular values >= 3e-4 end within 1e-3 of 1 and the
    result approaches the polar factor U V^T."""
    spec = GOLDEN["hybrid"]["value"]
    sched = [tuple(spec[0])] * spec[1] + [tuple(spec[2])] * spec[3]
    a, b, c = sched[-1]
    assert a + b + c == 1.0 and a + 3 * b + 5 * c == 0.0
    grid = np.geomspace(3e-4, 1.0, 100001)
    mapped = scalar_map(grid, sched, 10)
    assert mapped.min() >= 1.0 - 1e-9 and mapped.max() <= 1.001
    check_singular_value_map(O.newton_schulz, (20, 33), 10, sched)
    r = rng(11)
    g = r.standard_normal((24, 40))
    u, s, vt = np.linalg.svd(g, full_matrices=False)
    if (s / np.linalg.norm(s)).min() >= 3e-4:
        assert rel(O.newton_schulz(g, sched, 10, 0.0), u @ vt) <= 1e-3


# ---------------------------------------------------------------------------
# momentum, norm, normalisation, scale, apply, whole step
# ---------------------------------------------------------------------------
def test_momentum_closed_form():
    """Zero-initialised EMA momentum after t steps is
    (1 - mu) * sum_k mu^(t-k) G_k."""
    r = rng(12)
    mu = 0.95
    gs = [r.standard_normal((6, 7)) for _ in range(4)]
    m = np.zeros((6, 7))
    for t, g in enumerate(gs, 1):
        m = O.momentum_lerp(m, g, mu)
        want = (1 - mu) * sum(mu ** (t - k) * gs[k - 1] for k in range(1, t + 1))
        assert np.max(np.abs(m - want)) <= 1e-14


def test_momentum_forms_give_same_update():
    """The EMA form and [csdn]'s undamped sum differ by the factor (1 - mu)
    from a zero start, which normalisation removes (eps aside)."""
    r = rng(13)
    g1, g2 = r.standard_normal((16, 24)), r.standard_normal((16, 24))
    ema = O.momentum_lerp(O.momentum_lerp(np.zeros_like(g1), g1, 0.9), g2, 0.9)
    acc = 0.9 * g1 + g2
    assert rel(O.newton_schulz(ema, eps=0.0), O.newton_schulz(acc, eps=0.0)) <= 1e-13


def test_frobenius_norm_exact_sum():
    r = rng(14)
    m = r.standard_normal((9, 13)).astype(np.float32)
    want = math.sqrt(math.fsum(float(v) * float(v) for v in m.ravel()))
    assert abs(O.frobenius_norm(m) - want) <= 1e-15 * want
    big = r.standard_normal((300, 400))
    assert abs(O.frobenius_norm(big) ** 2 / big.size - 1.0) < 0.02


def test_normalise_bounds_spectrum():
    """Dividing by the Frobenius norm bounds the top singular value by 1
    ([csdn] section "1. Preprocessing")."""
    r = rng(15)
    for shape in ((10, 30), (30, 10), (25, 25)):
        g = r.standard_normal(shape) * 1e3
        x = O.normalise(g)
        assert np.linalg.norm(x, 2) <= 1.0
        assert abs(np.linalg.norm(x) - np.linalg.norm(g) / (np.linalg.norm(g) + 1e-7)) < 1e-15


def test_zero_gradient_gives_pure_decay():
    """A zero momentum matrix normalises to 0/(0 + eps) = 0: no update, only
    decay."""
    p = rng(16).standard_normal((8, 12))
    out = O.muon_step_matrix(p, np.zeros((8, 12)), np.zeros((8, 12)), lr=0.5, wd=0.5)
    assert np.all(out["o"] == 0.0) and out["nu"] == 0.0
    assert np.array_equal(out["p"], p * 0.75)


def test_missing_gradient_is_skipped():
    p = rng(17).standard_normal((4, 5))
    m = rng(18).standard_normal((4, 5))
    out = O.muon_step_matrix(p, None, m)
    assert np.array_equal(out["p"], p) and np.array_equal(out["m"], m) and out["o"] is None


def test_rms_scale_reading():
    assert O.rms_scale(1536, 80, "sqrt_max1") == math.sqrt(1536 / 80)
    assert O.rms_scale(80, 1536, "sqrt_max1") == 1.0
    assert O.rms_scale(8192, 28672, "sqrt_max1") == 1.0
    assert O.rms_scale(64, 64, "sqrt_max1") == 1.0
    assert O.rms_scale(1536, 80, None) == 1.0
    with pytest.raises(ValueError):
        O.rms_scale(2, 2, "bogus")


def test_apply_closed_form():
    """p <- p (1 - lr wd) - lr s O with binary-exact numbers."""
    p = np.full((3, 4), 2.0)
    o = np.arange(12.0).reshape(3, 4) / 8
    got = O.apply_update(p, o, lr=0.5, wd=0.5, scale=2.0)
    want = np.array([[2.0 * 0.75 - 0.5 * 2.0 * (i * 4 + j) / 8 for j in range(4)] for i in range(3)])
    assert np.array_equal(got, want)


def test_whole_step_order_and_stages():
    """The step is momentum, then NS of the new momentum, then the decayed
    update with the RMS scale of the stored shape."""
    r = rng(19)
    p, g, m = r.standard_normal((12, 5)), r.standard_normal((12, 5)), r.standard_normal((12, 5))
    out = O.muon_step_matrix(p, g, m, lr=0.1, mu=0.8, wd=0.2, rms_mode="sqrt_max1")
    m_new = 0.8 * m + 0.2 * g
    assert np.max(np.abs(out["m"] - m_new)) <= 1e-15
    assert abs(out["nu"] - np.linalg.norm(m_new)) <= 1e-14
    u, s, vt = np.linalg.svd(m_new, full_matrices=False)
    want_o = (u * scalar_map(s / (np.linalg.norm(s) + 1e-7), (QUINTIC,), 5)) @ vt
    assert rel(out["o"], want_o) <= 1e-12
    assert out["scale"] == math.sqrt(12 / 5)
    assert np.max(np.abs(out["p"] - (p * 0.98 - 0.1 * math.sqrt(12 / 5) * out["o"]))) <= 1e-15


def test_bad_inputs_rejected():
    with pytest.raises(ValueError):
        O.newton_schulz(np.ones(5))
    with pytest.raises(ValueError):
        O.newton_schulz(np.ones((3, 3)), coeffs=[QUINTIC, QUINTIC], steps=5)
