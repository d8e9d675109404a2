"""GPU edge cases: the longest side the ABI accepts, many tiny matrices in one
call, the largest step count with per-step coefficients over every kernel
class, calls where almost every gradient is absent, a non-finite gradient in
one matrix of a grouped call, and the transpose equivariance of the wide and
tall paths."""
import numpy as np
import pytest

import matrix_aware_optimizer_libmuon_amd as muon
from matrix_aware_optimizer_libmuon_amd import workloads as W
from oracle import muon_oracle as O
from tests.bf16_error import ns_error_estimate_for
from tests.bf16_model import newton_schulz_bf16
from tests.gpu_helpers import Run, check_apply_consistency, rel, say

pytestmark = pytest.mark.gpu

TOL_NS = 2e-2
TOL_F32 = 1e-5
MAX_DIM = 1 << 20


@pytest.mark.parametrize("shape", [(1, MAX_DIM), (MAX_DIM, 1)])
def test_longest_side_accepted(shape):
    """A single row (or column) of 2^20 elements: normalisation is exact up to
    rounding and every Newton-Schulz step keeps the vector's direction, so O is
    the normalised vector scaled by p^5(1) (the quintic's orbit of 1)."""
    mi = W.adhoc_inputs(*shape, "bf16", seed=1)
    run = Run([mi]).step(lr=0.02, mu=0.95, wd=0.0)
    out = O.muon_step_matrix(mi.param, mi.grad, mi.mom, lr=0.02, mu=0.95, wd=0.0)
    m_err = rel(run.mom(0), out["m"])
    o_err = rel(run.o(0), out["o"])
    say(f"  {shape}: M {m_err:.1e} O {o_err:.2e}")
    assert m_err <= TOL_F32 and o_err <= TOL_NS
    g = mi.grad.astype(np.float64)
    assert rel(run.o(0), 0.6964364095 * g / np.linalg.norm(g)) <= TOL_NS
    check_apply_consistency(run, 0, 0.02, 0.0, 1.0)


def test_thousands_of_tiny_matrices():
    """5000 matrices of at most 8 x 8 in one grouped call; every one is
    compared with the fp64 oracle.

    Pass condition per matrix: relative Frobenius error of O at most
    max(2e-2, 4 e), where e is the first-order RMS size of the bf16 rounding
    error of the documented rounding points propagated through the
    iteration, computed from the oracle's own spectrum of the normalised
    momentum (tests/bf16_error.py).  Inside the domain e <= 5e-3 this is the
    plain 2e-2 bar.  Tiny matrices whose normalised singular values sit where
    the five-step quintic map is steep (slope up to a^5 ~ 486 near 0) have an
    O that bf16 cannot determine to 2e-2 at all; there the bar follows the
    method's own precision, never the library's output.  Momentum (1e-5) and
    the apply stage (1e-5, against the library's own O) are checked for every
    matrix as well, and every O's singular values stay within the quintic's
    spectral bound 1.2024 (+0.03)."""
    rng = np.random.default_rng(3)
    shapes = [(int(rng.integers(1, 9)), int(rng.integers(1, 9))) for _ in range(5000)]
    inputs = [W.adhoc_inputs(r, c, "f32", seed=10 + k) for k, (r, c) in enumerate(shapes)]
    run = Run(inputs).step(lr=0.02, mu=0.95, wd=0.01)
    errs, ests, beyond, model_dev = [], [], 0, 0.0
    for i, mi in enumerate(inputs):
        out = O.muon_step_matrix(mi.param, mi.grad, mi.mom, lr=0.02, mu=0.95, wd=0.01)
        o = run.o(i)
        err = rel(o, out["o"])
        est = ns_error_estimate_for(out["m"], (O.QUINTIC,), 5)
        errs.append(err)
        ests.append(est)
        assert rel(run.mom(i), out["m"]) <= TOL_F32, (i, shapes[i])
        check_apply_consistency(run, i, 0.02, 0.01, 1.0)
        assert np.linalg.norm(o, 2) <= 1.2024 + 0.03, (i, shapes[i])
        assert err <= max(TOL_NS, 4.0 * est), (i, shapes[i], err, est)
        if err > TOL_NS:
            beyond += 1
            # diagnostic only: distance to a numpy emulation of the same
            # rounding points (not a pass condition)
            model_dev = max(model_dev, rel(o, newton_schulz_bf16(out["m"], (O.QUINTIC,), 5)))
    errs, ests = np.array(errs), np.array(ests)
    inside = ests <= TOL_NS / 4
    say(f"  5000 tiny matrices: O error max {errs.max():.2e}, median {np.median(errs):.2e}; "
        f"error / estimate max {np.max(errs / np.maximum(ests, 1e-30)):.2f}, "
        f"median {np.median(errs / np.maximum(ests, 1e-30)):.2f}; {int(inside.sum())} inside "
        f"the 2e-2 domain; {beyond} beyond 2e-2 (estimate there >= {ests[errs > TOL_NS].min() if beyond else 0:.2e}; "
        f"max distance to the bf16 emulation {model_dev:.1e})")


def test_sixty_four_steps_with_per_step_coefficients_over_every_class():
    """ns = 64 (the maximum) with a different coefficient triple per step, on
    a fused, a 128-tile and a 256-tile matrix in one call."""
    steps = 64
    coeffs = [O.QUINTIC if k % 3 else (1.5, -0.5, 0.0) for k in range(steps)]
    shapes = [(40, 300), (300, 200), (1024, 1100)]
    inputs = [W.adhoc_inputs(r, c, "bf16", seed=20 + k) for k, (r, c) in enumerate(shapes)]
    run = Run(inputs).step(lr=0.02, mu=0.95, wd=0.0, ns_steps=steps, coeffs=coeffs)
    for i, mi in enumerate(inputs):
        out = O.muon_step_matrix(mi.param, mi.grad, mi.mom, lr=0.02, mu=0.95, wd=0.0,
                                 ns_steps=steps, coeffs=coeffs)
        err = rel(run.o(i), out["o"])
        say(f"  {shapes[i]}: O {err:.2e} after {steps} steps")
        assert err <= TOL_NS


def test_only_one_gradient_present():
    shapes = [(64, 64), (300, 200), (1024, 1024), (48, 1536), (1536, 80)]
    inputs = [W.adhoc_inputs(r, c, "bf16", seed=30 + k, mom_std=0.1) for k, (r, c) in enumerate(shapes)]
    present = [False, False, True, False, False]
    run = Run(inputs, grads_present=present).step(lr=0.02, mu=0.95, wd=0.1)
    for i, mi in enumerate(inputs):
        if present[i]:
            out = O.muon_step_matrix(mi.param, mi.grad, mi.mom, lr=0.02, mu=0.95, wd=0.1)
            assert rel(run.o(i), out["o"]) <= TOL_NS
        else:
            assert np.array_equal(run.param(i), mi.param) and np.array_equal(run.mom(i), mi.mom)


# two matrices per kernel class, wide then tall: fused (short side <= 128 and
# fits LDS), 128-tile, 256-tile
_CLASS_SHAPES = {"fused": [(64, 96), (96, 64)], "128": [(256, 768), (768, 256)],
                 "256": [(1024, 1536), (1536, 1024)]}
_BF16_BITS = {"nan": 0x7FC0, "inf": 0x7F80}


@pytest.mark.parametrize("bad", ["nan", "inf"])
@pytest.mark.parametrize("cls", ["fused", "128", "256"])
def test_nonfinite_gradient_stays_in_its_matrix(cls, bad):
    """One NaN (or +inf) gradient entry in one matrix of a grouped step.  The
    pages say nothing of it; the plain reading is that the arithmetic carries
    it: that matrix's momentum is non-finite at that entry only, its norm is
    non-finite, and NS spreads NaN over its whole O and update, as in the fp64
    oracle.  Every other matrix of the same launches, in its class and in the
    others, matches the oracle: the grouped launches keep the matrices' tiles,
    norm slots and buffers apart."""
    lr, mu, wd = 0.02, 0.95, 0.01
    shapes = [s for k in ("fused", "128", "256") for s in _CLASS_SHAPES[k]]
    inputs = [W.adhoc_inputs(r, c, "bf16", seed=70 + i) for i, (r, c) in enumerate(shapes)]
    b = shapes.index(_CLASS_SHAPES[cls][0])
    mi = inputs[b]
    r0, c0 = mi.rows // 2, mi.cols // 3
    mi.grad_bits[r0, c0] = _BF16_BITS[bad]
    mi.grad[r0, c0] = np.float32(np.nan if bad == "nan" else np.inf)
    run = Run(inputs).step(lr=lr, mu=mu, wd=wd)
    for i, m in enumerate(inputs):
        out = O.muon_step_matrix(m.param, m.grad, m.mom, lr=lr, mu=mu, wd=wd)
        if i == b:
            mom = run.mom(i)
            np.testing.assert_array_equal(np.isfinite(mom), np.isfinite(out["m"]))
            fin = np.isfinite(out["m"])
            assert fin.sum() == mom.size - 1
            assert rel(mom[fin], out["m"][fin]) <= TOL_F32
            assert not np.isfinite(run.nu(i))
            assert np.isnan(out["o"]).all() and np.isnan(run.o(i)).all()
            assert np.isnan(run.param(i)).all()
            say(f"  {cls}/{bad}: matrix {i} {shapes[i]} non-finite as the oracle")
        else:
            assert np.isfinite(run.o(i)).all() and np.isfinite(run.param(i)).all()
            assert rel(run.mom(i), out["m"]) <= TOL_F32
            assert rel(run.o(i), out["o"]) <= TOL_NS
            check_apply_consistency(run, i, lr, wd, 1.0)


@pytest.mark.parametrize("cls", ["fused", "128", "256"])
def test_transpose_equivariance(cls):
    """NS(G^T) = NS(G)^T ([wmrh] 2.2: the iteration acts on singular values;
    the transpose rule of [airosetta] newtonschulz5 runs it on the short side
    either way).  G and G^T in one grouped call take different operand paths:
    the wide matrix is read K-contiguous, the tall one through the transposing
    LDS reads, and its X update is the swapped product X^T C.  Both paths
    round at the same points and sum the same terms in the same K order (one
    MFMA per 32-deep slice, operands exchanged on the tall path), and the
    norm's scale is one fp32 value per matrix, so the outputs are the exact
    transposes of each other (measured so for every class; any difference
    would mean the two paths compute different sums)."""
    lr, mu, wd = 0.02, 0.95, 0.01
    r, c = _CLASS_SHAPES[cls][0]
    g = W.adhoc_inputs(r, c, "bf16", seed=90, mom_std=0.5)
    gt = W.MatrixInputs(c, r, np.ascontiguousarray(g.grad.T), np.ascontiguousarray(g.grad_bits.T),
                        np.ascontiguousarray(g.param.T), np.ascontiguousarray(g.mom.T))
    run = Run([g, gt]).step(lr=lr, mu=mu, wd=wd)
    assert np.array_equal(run.mom(1), run.mom(0).T)
    o, ot = run.o(0), run.o(1)
    same = np.array_equal(ot, o.T)
    err = rel(ot, o.T)
    say(f"  {cls} {r}x{c}: O(G^T) vs O(G)^T rel {err:.3e}, bit-identical {same}")
    assert same, f"O(G^T) differs from O(G)^T: rel {err:.3e}"
    assert np.array_equal(run.param(1), run.param(0).T)


def test_check_finite_names_the_matrix(monkeypatch):
    """MUON_CHECK_FINITE: the step reads back the momentum norms and fails
    with MUON_ENONFINITE naming the first matrix whose norm is NaN or
    infinite, for an eager step and a plan step; the step itself has run (the
    other matrices match the oracle); a clean list passes; unset, the same
    call succeeds."""
    import torch

    lr, mu, wd = 0.02, 0.95, 0.01
    shapes = [(64, 96), (256, 768), (1024, 1536), (768, 256)]
    inputs = [W.adhoc_inputs(r, c, "bf16", seed=130 + i) for i, (r, c) in enumerate(shapes)]
    bad = 2
    inputs[bad].grad_bits[5, 7] = _BF16_BITS["nan"]
    inputs[bad].grad[5, 7] = np.float32(np.nan)
    monkeypatch.setenv("MUON_CHECK_FINITE", "1")
    run = Run(inputs)
    with pytest.raises(muon.LibMuonError) as ei:
        run.step(lr=lr, mu=mu, wd=wd)
    torch.cuda.synchronize()
    assert ei.value.status == muon.MUON_ENONFINITE and f"matrix {bad}:" in str(ei.value), str(ei.value)
    say(f"  eager: {ei.value}")
    for i, mi in enumerate(inputs):
        if i != bad:
            out = O.muon_step_matrix(mi.param, mi.grad, mi.mom, lr=lr, mu=mu, wd=wd)
            assert rel(run.o(i), out["o"]) <= TOL_NS
    # a plan step over the same buffers reports it too
    plan = muon.Plan(run.p, run.g, run.m, lr=lr, mu=mu, wd=wd, workspace=run.ws)
    with pytest.raises(muon.LibMuonError) as ei:
        plan.step()
    torch.cuda.synchronize()
    assert ei.value.status == muon.MUON_ENONFINITE and f"matrix {bad}:" in str(ei.value)
    plan.close()
    # a clean list passes with the check on, and the NaN list passes with it off
    clean = [W.adhoc_inputs(r, c, "bf16", seed=140 + i) for i, (r, c) in enumerate(shapes)]
    Run(clean).step(lr=lr, mu=mu, wd=wd)
    monkeypatch.delenv("MUON_CHECK_FINITE")
    Run(inputs).step(lr=lr, mu=mu, wd=wd)
