"""GPU edge cases: the longest side the ABI accepts, many tiny matrices in one
call, the largest step count with per-step coefficients over every kernel
class, and calls where almost every gradient is absent."""
import numpy as np
import pytest

import matrix_aware_optimizer_libmuon_amd as muon
from matrix_aware_optimizer_libmuon_amd import workloads as W
from oracle import muon_oracle as O
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
    """5000 matrices of at most 8 x 8.  A few such matrices have a normalised
    singular value near 2e-3, where five quintic steps amplify the bf16
    rounding of X itself past 2e-2 of the fp64 result; there the GPU must match
    the bf16 rounding model instead (it does to the last bit on these sizes),
    which shows the excess is the method's precision, not a kernel fault."""
    rng = np.random.default_rng(3)
    shapes = [(int(rng.integers(1, 9)), int(rng.integers(1, 9))) for _ in range(5000)]
    inputs = [W.adhoc_inputs(r, c, "f32", seed=10 + k) for k, (r, c) in enumerate(shapes)]
    run = Run(inputs).step(lr=0.02, mu=0.95, wd=0.01)
    worst, within = 0.0, 0
    sampled = range(0, len(shapes), 97)
    for i in sampled:
        mi = inputs[i]
        out = O.muon_step_matrix(mi.param, mi.grad, mi.mom, lr=0.02, mu=0.95, wd=0.01)
        err = rel(run.o(i), out["o"])
        worst = max(worst, err)
        assert rel(run.mom(i), out["m"]) <= TOL_F32
        check_apply_consistency(run, i, 0.02, 0.01, 1.0)
        if err <= TOL_NS:
            within += 1
        else:
            model = newton_schulz_bf16(out["m"], (O.QUINTIC,), 5)
            assert rel(run.o(i), model) <= 1e-3, (shapes[i], err)
    say(f"  5000 tiny matrices: worst sampled O error {worst:.2e}; {within} of {len(sampled)} within 2e-2")
    assert within >= 0.9 * len(sampled)


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
