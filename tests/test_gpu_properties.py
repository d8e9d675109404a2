"""Properties of the step that fix results exactly, and the per-matrix update
scale of the boundary, on the GPU."""
import numpy as np
import pytest

from matrix_aware_optimizer_libmuon_amd import workloads as W
from oracle import muon_oracle as O
from tests.gpu_helpers import Run, check_apply_consistency, rel, say

pytestmark = pytest.mark.gpu

TOL_NS = 2e-2
TOL_F32 = 1e-5
# one wide shape per kernel class: fused (short side <= 128, fits LDS),
# 128-tile, 256-tile
CLASS_SHAPES = {"fused": (64, 96), "128": (256, 768), "256": (1024, 1536)}


def _scaled(mi: W.MatrixInputs, k: int) -> W.MatrixInputs:
    """The same matrix with gradient and momentum multiplied by 2^k (exact in
    bf16 and fp32 away from overflow and underflow)."""
    f = np.float32(2.0 ** k)
    g = (mi.grad * f).astype(np.float32)
    bits = (g.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), g)
    return W.MatrixInputs(mi.rows, mi.cols, g, bits, mi.param.copy(), (mi.mom * f).astype(np.float32))


@pytest.mark.parametrize("cls", ["fused", "128", "256"])
def test_scale_invariance_is_exact_without_eps(cls):
    """NS(cG) = NS(G) for c > 0 ([wmrh] 2.2: the iteration sees only the
    normalised matrix).  With eps = 0 and c a power of two every stage before
    the first rounding scales exactly: M by c, the norm by c, so M / norm and
    everything after it are the same bits.  Gradient and momentum scaled by
    2^3 and 2^-5 ride in one call with the original: bit-identical O and
    updates, norms in the exact ratio."""
    lr, mu, wd = 0.02, 0.95, 0.01
    r, c = CLASS_SHAPES[cls]
    base = W.adhoc_inputs(r, c, "bf16", seed=110, mom_std=0.5)
    inputs = [base, _scaled(base, 3), _scaled(base, -5)]
    run = Run(inputs).step(lr=lr, mu=mu, wd=wd, eps=0.0)
    o0, nu0 = run.o(0), run.nu(0)
    for i, k in ((1, 3), (2, -5)):
        assert np.array_equal(run.o(i), o0), f"2^{k}: O differs, rel {rel(run.o(i), o0):.3e}"
        assert np.array_equal(run.param(i), run.param(0))
        assert abs(run.nu(i) / nu0 - 2.0 ** k) <= 1e-14 * 2.0 ** k
    out = O.muon_step_matrix(base.param, base.grad, base.mom, lr=lr, mu=mu, wd=wd, eps=0.0)
    err = rel(o0, out["o"])
    say(f"  {cls} {r}x{c}: scaled copies bit-identical; O vs oracle {err:.3e}")
    assert err <= TOL_NS


def test_per_matrix_scale_overrides_the_call_mode():
    """muon_matrix_t.scale: a value > 0 is the matrix's update scale s; 0 (or
    none) leaves s to the call's rms_scale mode, here sqrt(max(1, rows/cols))
    ([csdn] "3. Scaling and update" asks for a size-dependent rescale; the
    formula is the reading taken).  O does not depend on s; only the apply
    stage does."""
    lr, mu, wd = 0.02, 0.95, 0.01
    shapes = [(1536, 80), (64, 96), (256, 768), (768, 256), (1024, 1536), (96, 64)]
    scales = [None, 0.5, None, 2.5, 0.0, 3.0]
    inputs = [W.adhoc_inputs(r, c, "bf16", seed=120 + i) for i, (r, c) in enumerate(shapes)]
    run = Run(inputs).step(lr=lr, mu=mu, wd=wd, ns_steps=5, rms_scale="sqrt_max1", scales=scales)
    for i, (mi, s) in enumerate(zip(inputs, scales)):
        out = O.muon_step_matrix(mi.param, mi.grad, mi.mom, lr=lr, mu=mu, wd=wd,
                                 rms_mode="sqrt_max1")
        want_s = s if s else out["scale"]
        assert rel(run.mom(i), out["m"]) <= TOL_F32
        assert rel(run.o(i), out["o"]) <= TOL_NS
        ap = check_apply_consistency(run, i, lr, wd, want_s)
        say(f"  {shapes[i]}: s {want_s:.4f} ({'override' if s else 'mode'}), apply {ap:.1e}")
    # the mode's value really differs from the overrides on the tall matrices
    assert O.rms_scale(1536, 80, "sqrt_max1") > 4.0 and O.rms_scale(768, 256, "sqrt_max1") > 1.7
