"""GPU parity of the fused small-matrix iteration (every Newton-Schulz step
of a matrix in one workgroup, X, A and C in LDS) against the fp64 oracle:
wide and tall shapes up to the LDS limit, the iterate buffers after 0 to 3
steps, per-step coefficients, and a launch over many ragged small matrices.
Tolerances as for the tiled path: 2e-2 relative Frobenius on O, 1e-5 on the
fp32 stages."""
import numpy as np
import pytest
import torch

import matrix_aware_optimizer_libmuon_amd as muon
from matrix_aware_optimizer_libmuon_amd import workloads as W
from oracle import muon_oracle as O
from tests.gpu_helpers import DEV, Run, check_apply_consistency, rel, say

pytestmark = pytest.mark.gpu

TOL_NS = 2e-2
TOL_F32 = 1e-5

# every one takes the fused kernel (checked first); the last five sit at the
# 160 KB LDS limit
FUSED = [(1, 1), (2, 3), (40, 1), (17, 15), (33, 65), (64, 64), (96, 200), (128, 128),
         (256, 128), (100, 300), (300, 100), (64, 1024), (1024, 64), (32, 2304)]


def _is_fused(shape):
    return muon.workspace_view([shape], 0, 5)["tile"] == 32


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_shapes_match_oracle(dtype):
    assert all(_is_fused(s) for s in FUSED)
    lr, mu, wd = 0.02, 0.9, 0.05
    inputs = [W.adhoc_inputs(r, c, dtype, seed=700 + k, mom_std=0.3) for k, (r, c) in enumerate(FUSED)]
    run = Run(inputs).step(lr=lr, mu=mu, wd=wd, ns_steps=5, rms_scale="sqrt_max1")
    for i, mi in enumerate(inputs):
        out = O.muon_step_matrix(mi.param, mi.grad, mi.mom, lr=lr, mu=mu, wd=wd, ns_steps=5,
                                 rms_mode="sqrt_max1")
        m_err = rel(run.mom(i), out["m"])
        nu_err = abs(run.nu(i) - out["nu"]) / out["nu"]
        o_err = rel(run.o(i), out["o"])
        ap = check_apply_consistency(run, i, lr, wd, out["scale"])
        say(f"  fused {mi.rows}x{mi.cols} {dtype}: M {m_err:.1e} nu {nu_err:.1e} O {o_err:.3e} apply {ap:.1e}")
        assert m_err <= TOL_F32 and nu_err <= TOL_F32 and o_err <= TOL_NS


@pytest.mark.parametrize("shape", [(48, 200), (200, 48)])
def test_fused_iterate_buffers_after_k_steps(shape):
    """After k steps the final iterate sits in buffer k & 1 and the one
    before it in the other buffer, as for the tiled kernels."""
    r, c = shape
    mi = W.adhoc_inputs(r, c, "bf16", seed=800)
    x = O.normalise(O.momentum_lerp(mi.mom, mi.grad, 0.95))
    for k in range(4):
        run = Run([mi]).step(lr=0.02, mu=0.95, wd=0.0, ns_steps=k)
        o = run.o(0)
        ref = O.newton_schulz(mi.grad, (O.QUINTIC,), k) if k else x
        assert rel(o, ref) <= TOL_NS, (k, rel(o, ref))
        if k >= 1:
            prev = run.x(0, (k - 1) & 1)[:r, :c]
            ref_prev = O.newton_schulz(mi.grad, (O.QUINTIC,), k - 1) if k > 1 else x
            assert rel(prev, ref_prev) <= TOL_NS, (k, rel(prev, ref_prev))
        say(f"  {shape} k={k}: O {rel(o, ref):.2e}")


def test_fused_per_step_coefficients():
    g = W.adhoc_inputs(64, 448, "f32", seed=810).grad
    assert _is_fused((64, 448))
    (out,) = muon.orthogonalize([torch.from_numpy(g).to(DEV)], ns_steps=10, coeffs=muon.HYBRID)
    ref = O.newton_schulz(g, [O.QUINTIC] * 8 + [O.HYBRID_TAIL] * 2, 10)
    err = rel(out.float().cpu().numpy(), ref)
    say(f"  fused hybrid schedule: {err:.3e}")
    assert err <= TOL_NS


def test_many_ragged_small_matrices_in_one_call():
    """600 matrices, rows and cols uniform on {1..128} x {1..512}: fused and
    tiled ones mixed in one call; a sample is checked against the oracle."""
    rng = np.random.default_rng(5)
    shapes = [(int(rng.integers(1, 129)), int(rng.integers(1, 513))) for _ in range(600)]
    shapes = [s if k % 2 else s[::-1] for k, s in enumerate(shapes)]
    inputs = [W.adhoc_inputs(r, c, "bf16", seed=900 + k) for k, (r, c) in enumerate(shapes)]
    run = Run(inputs).step(lr=0.02, mu=0.95, wd=0.01, ns_steps=5)
    nf = sum(_is_fused(s) for s in shapes)
    say(f"  {nf} of {len(shapes)} fused")
    worst = 0.0
    for i in range(0, len(shapes), 7):
        mi = inputs[i]
        out = O.muon_step_matrix(mi.param, mi.grad, mi.mom, lr=0.02, mu=0.95, wd=0.01, ns_steps=5)
        err = rel(run.o(i), out["o"])
        worst = max(worst, err)
        assert err <= TOL_NS, (shapes[i], err)
        check_apply_consistency(run, i, 0.02, 0.01, 1.0)
    say(f"  worst sampled O error {worst:.3e}")
