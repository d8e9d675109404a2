"""GPU parity of libmuon against the fp64 oracle on seeded inputs, edge
shapes, grouped dispatch, and stage-by-stage consistency of the kernels.

Tolerances (relative Frobenius, per matrix): momentum and norm 1e-5 (fp32
path), the bf16 Newton-Schulz output O 2e-2, the apply stage 1e-5 against
the library's own O."""
import math

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

EDGE_SHAPES = [(1, 1), (1, 40), (40, 1), (15, 17), (17, 15), (16, 16), (48, 80), (80, 48),
               (100, 300), (300, 100), (128, 128), (129, 257), (257, 129), (256, 768), (640, 200)]


def _compare(run, i, mi, out, lr, wd, scale):
    m_err = rel(run.mom(i), out["m"])
    nu_err = abs(run.nu(i) - out["nu"]) / out["nu"]
    o_err = rel(run.o(i), out["o"])
    ap = check_apply_consistency(run, i, lr, wd, scale)
    assert m_err <= TOL_F32, f"momentum {m_err}"
    assert nu_err <= TOL_F32, f"norm {nu_err}"
    assert o_err <= TOL_NS, f"O {o_err}"
    return m_err, nu_err, o_err, ap


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_edge_shapes_match_oracle(dtype):
    lr, mu, wd = 0.02, 0.9, 0.1
    inputs = [W.adhoc_inputs(r, c, dtype, seed=k, mom_std=0.3) for k, (r, c) in enumerate(EDGE_SHAPES)]
    say(f"edge shapes {dtype}: {EDGE_SHAPES}")
    run = Run(inputs).step(lr=lr, mu=mu, wd=wd, ns_steps=5, rms_scale="sqrt_max1")
    for i, mi in enumerate(inputs):
        out = O.muon_step_matrix(mi.param, mi.grad, mi.mom, lr=lr, mu=mu, wd=wd, ns_steps=5,
                                 rms_mode="sqrt_max1")
        errs = _compare(run, i, mi, out, lr, wd, out["scale"])
        say(f"  {mi.rows}x{mi.cols}: M {errs[0]:.2e} nu {errs[1]:.2e} O {errs[2]:.2e} apply {errs[3]:.2e}")


def test_single_fp32_gradient_256x768():
    """The single-gradient workload: fp32 256 x 768, N(0,1), zero momentum,
    mu 0.95, lr 0.02, wd 0, eps 1e-7, 5 quintic steps."""
    w = W.WORKLOADS[1]
    mi = W.matrix_inputs(w, 0)
    run = Run([mi]).step(lr=w.lr, mu=w.mu, wd=w.wd, ns_steps=w.ns_steps, eps=w.eps)
    out = O.muon_step_matrix(mi.param, mi.grad, mi.mom, lr=w.lr, mu=w.mu, wd=w.wd,
                             ns_steps=w.ns_steps, eps=w.eps)
    errs = _compare(run, 0, mi, out, w.lr, w.wd, 1.0)
    say(f"workload 1: M {errs[0]:.2e} nu {errs[1]:.2e} O {errs[2]:.2e} apply {errs[3]:.2e}")
    # the output spectrum sits in the quintic band
    sv = np.linalg.svd(run.o(0).astype(np.float64), compute_uv=False)
    assert 0.68 - 0.03 <= sv.min() and sv.max() <= 1.2024 + 0.03


def test_cubic_thirty_steps_reaches_polar_factor():
    """With the cubic coefficients (1.5, -0.5, 0) and 30 steps the bf16
    iteration lands on the SVD's U V^T within the bf16 budget."""
    w = W.WORKLOADS[1]
    g, _ = W.grad(w, 0, 0)
    x = torch.from_numpy(g).to(DEV)
    (out,) = muon.orthogonalize([x], ns_steps=30, coeffs=(1.5, -0.5, 0.0))
    u, s, vt = np.linalg.svd(g.astype(np.float64), full_matrices=False)
    err = rel(out.float().cpu().numpy(), u @ vt)
    ref = O.newton_schulz(g, (O.CUBIC,), 30)
    say(f"cubic x30 vs UV^T: {err:.3e}; oracle vs UV^T {rel(ref, u @ vt):.1e}")
    assert err <= TOL_NS


def test_zero_gradient_and_skipped_matrices():
    lr, wd = 0.5, 0.25
    z = W.adhoc_inputs(64, 96, "bf16", seed=1)
    z.grad[:] = 0
    z.grad_bits[:] = 0
    live = W.adhoc_inputs(96, 64, "bf16", seed=2)
    skip = W.adhoc_inputs(80, 80, "f32", seed=3, mom_std=1.0)
    run = Run([z, live, skip], grads_present=[True, True, False]).step(lr=lr, mu=0.95, wd=wd)
    assert np.all(run.o(0) == 0.0) and run.nu(0) == 0.0
    decay = np.float32(1.0) - np.float32(lr) * np.float32(wd)
    assert np.array_equal(run.param(0), z.param * decay)          # pure decay, exact in fp32
    assert np.array_equal(run.param(2), skip.param) and np.array_equal(run.mom(2), skip.mom)
    out = O.muon_step_matrix(live.param, live.grad, live.mom, lr=lr, mu=0.95, wd=wd)
    assert rel(run.o(1), out["o"]) <= TOL_NS


def test_grouped_dispatch_equals_one_by_one_and_is_order_free():
    shapes = [(48, 1536), (1536, 80), (256, 256), (64, 512), (512, 64), (300, 700)]
    inputs = [W.adhoc_inputs(r, c, "bf16", seed=10 + k, mom_std=0.1) for k, (r, c) in enumerate(shapes)]
    kw = dict(lr=0.02, mu=0.95, wd=0.01, ns_steps=5)
    grouped = Run(inputs).step(**kw)
    alone = [Run([mi]).step(**kw) for mi in inputs]
    perm = [3, 0, 5, 1, 4, 2]
    shuffled = Run([inputs[j] for j in perm]).step(**kw)
    for i in range(len(shapes)):
        a = grouped.o(i)
        b = alone[i].o(0)
        c = shuffled.o(perm.index(i))
        same_ab = np.mean(a == b)
        same_ac = np.mean(a == c)
        say(f"  {shapes[i]}: identical fraction alone {same_ab:.6f} permuted {same_ac:.6f}")
        # identical up to the order of the fp64 atomic norm accumulation
        assert rel(a, b) <= 1e-6 and rel(a, c) <= 1e-6
        assert np.array_equal(grouped.param(i), alone[i].param(0)) or rel(grouped.param(i), alone[i].param(0)) <= 1e-7


@pytest.mark.parametrize("shape", [(200, 300), (300, 200), (256, 256), (40, 600), (600, 100),
                                   (1024, 1536), (1536, 1024), (1100, 1100),
                                   (17, 15), (300, 100), (64, 1024)])
def test_stage_consistency_of_the_gemm_kernels(shape):
    """One iteration (ns = 1) read stage by stage from the workspace: every
    bf16 result is the round-to-nearest of the exact value computed from the
    library's own bf16 operands, up to fp32 accumulation error:
        A = X0 X0^T,  C = a I + b A + c A A (+ its low part when the short
        side is <= 128),  X1 = C X0 (= (C_hi + C_lo) X0).
    A and C are exactly symmetric; padding stays zero."""
    r, c = shape
    a_, b_, c_ = muon.QUINTIC
    mi = W.adhoc_inputs(r, c, "bf16", seed=21)
    run = Run([mi]).step(lr=0.02, mu=0.95, wd=0.0, ns_steps=1)
    v = run.view(0)
    m = min(r, c)
    x0 = run.x(0, 0).astype(np.float64)
    x1 = run.x(0, 1).astype(np.float64)
    A = run.a(0).astype(np.float64)
    C = run.c(0).astype(np.float64)
    C_lo = run.c_lo(0)
    assert (C_lo is not None) == (m <= 128)
    assert np.array_equal(A, A.T) and np.array_equal(C, C.T)
    tall = r > c
    X = x0.T if tall else x0            # logical m x n view (padded)
    Xn = x1.T if tall else x1
    u = 2.0 ** -8                       # bf16 unit roundoff (round to nearest)
    g = 2.0 ** -22                      # 4x the fp32 unit roundoff, per accumulated term
    K = X.shape[1]
    exact_A = X @ X.T
    bound_A = u * np.abs(exact_A) + g * K * (np.abs(X) @ np.abs(X).T)
    assert np.all(np.abs(A - exact_A) <= bound_A + 1e-30), "Gram"
    # a sits on the whole padded diagonal; harmless, since X's padding is zero
    exact_C = a_ * np.eye(A.shape[0]) + b_ * A + c_ * (A @ A)
    acc_C = g * (A.shape[0] * abs(c_) * (np.abs(A) @ np.abs(A)) + np.abs(b_ * A) + abs(a_))
    if C_lo is None:
        assert np.all(np.abs(C - exact_C) <= u * np.abs(exact_C) + acc_C + 1e-30), "C epilogue"
        Cfull = C
    else:
        C_lo = C_lo.astype(np.float64)
        assert np.array_equal(C_lo, C_lo.T)
        Cfull = C + C_lo                  # hi + lo carries ~16 significant bits
        assert np.all(np.abs(Cfull - exact_C) <= 2.0 ** -16 * np.abs(exact_C) + acc_C + 1e-30), "C pair"
        assert np.all(np.abs(C_lo) <= 2.0 ** -8 * np.abs(C) + 1e-30)
    exact_X = Cfull @ X
    bound_X = u * np.abs(exact_X) + g * 2 * Cfull.shape[0] * (np.abs(Cfull) @ np.abs(X))
    assert np.all(np.abs(Xn - exact_X) <= bound_X + 1e-30), "X update"
    # zero padding outside the m x n block is preserved by every stage
    assert np.all(A[m:, :] == 0) and np.all(A[:, m:] == 0)
    assert np.all(x1[r:, :] == 0) and np.all(x1[:, c:] == 0) and np.all(x0[r:, :] == 0)
    assert np.all(x0[:, c:] == 0)
    say(f"  {shape}: pads {v['rows_pad']}x{v['cols_pad']} m_pad {v['m_pad']} split {C_lo is not None} ok")


def test_orthogonalize_ns0_is_round_to_nearest_of_normalised_input():
    g = W.adhoc_inputs(333, 129, "f32", seed=30, grad_std=3.0).grad
    (out,) = muon.orthogonalize([torch.from_numpy(g).to(DEV)], ns_steps=0)
    got = out.float().cpu().numpy().astype(np.float64)
    x = O.normalise(g)
    # round to nearest: within half an ulp of x's binade (bf16 keeps 8
    # significant bits); truncation would reach a whole ulp
    half_ulp = np.exp2(np.floor(np.log2(np.abs(x))) - 8)
    err = np.abs(got - x)
    assert np.all(err <= half_ulp * (1 + 2.0 ** -12))
    assert np.mean(err > 0.5 * half_ulp) < 0.6


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_orthogonalize_matches_oracle(dtype):
    shapes = [(256, 768), (768, 256), (100, 100), (1536, 80)]
    xs = [W.adhoc_inputs(r, c, dtype, seed=40 + k).grad for k, (r, c) in enumerate(shapes)]
    dev = [torch.from_numpy(x).to(DEV) if dtype == "f32" else torch.from_numpy(x).to(DEV).bfloat16()
           for x in xs]
    outs = muon.orthogonalize(dev, ns_steps=5)
    for x, y in zip(xs, outs):
        err = rel(y.float().cpu().numpy(), O.newton_schulz(x))
        say(f"  orthogonalize {x.shape} {dtype}: {err:.3e}")
        assert err <= TOL_NS


def test_hybrid_schedule_per_step_coefficients():
    """Ten steps with per-step coefficients (8 quintic + 2 of (2, -1.5, 0.5))
    against the oracle, and the result is close to U V^T."""
    g = W.adhoc_inputs(192, 448, "f32", seed=50).grad
    (out,) = muon.orthogonalize([torch.from_numpy(g).to(DEV)], ns_steps=10, coeffs=muon.HYBRID)
    got = out.float().cpu().numpy()
    ref = O.newton_schulz(g, [O.QUINTIC] * 8 + [O.HYBRID_TAIL] * 2, 10)
    u, s, vt = np.linalg.svd(g.astype(np.float64), full_matrices=False)
    err, err_polar = rel(got, ref), rel(got, u @ vt)
    say(f"  hybrid: vs oracle {err:.3e}, vs UV^T {err_polar:.3e}")
    assert err <= TOL_NS and err_polar <= TOL_NS


def test_checkpoint_resume_equals_straight_run():
    """Step, copy the momentum and params out and back in, step again: the
    result equals two steps run straight (the only state is caller-owned)."""
    shapes = [(128, 384), (384, 128)]
    ins = [W.adhoc_inputs(r, c, "bf16", seed=60 + k) for k, (r, c) in enumerate(shapes)]
    ins2 = [W.adhoc_inputs(r, c, "bf16", seed=70 + k) for k, (r, c) in enumerate(shapes)]
    kw = dict(lr=0.02, mu=0.95, wd=0.01)
    a = Run(ins).step(**kw)
    a.set_grads(ins2)
    a.step(**kw)
    b = Run(ins).step(**kw)
    saved = [(b.p[i].cpu().clone(), b.m[i].cpu().clone()) for i in range(2)]
    c = Run(ins)
    for i in range(2):
        c.p[i].copy_(saved[i][0].to(DEV))
        c.m[i].copy_(saved[i][1].to(DEV))
    c.set_grads(ins2)
    c.step(**kw)
    for i in range(2):
        assert rel(c.param(i), a.param(i)) <= 1e-7 and rel(c.mom(i), a.mom(i)) <= 1e-7


def test_graph_capture_is_refused_before_anything_runs():
    """A call on a capturing stream returns MUON_ECAPTURE and leaves the
    parameters alone (the graph is ended, never replayed)."""
    mi = W.adhoc_inputs(64, 96, "bf16", seed=60)
    p = torch.from_numpy(mi.param).to(DEV)
    m = torch.from_numpy(mi.mom).to(DEV)
    g = torch.from_numpy(mi.grad_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    ws = muon.alloc_workspace([(64, 96)], DEV)
    x = torch.zeros(4, device=DEV)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    err = None
    with torch.cuda.stream(side):
        graph.capture_begin()
        try:
            x.add_(1.0)                      # something to capture besides the refused call
            muon.muon_step([p], [g], [m], workspace=ws)
        except muon.LibMuonError as e:
            err = e
        finally:
            graph.capture_end()
    torch.cuda.synchronize()
    assert err is not None and err.status == muon.MUON_ECAPTURE
    assert np.array_equal(p.cpu().numpy(), mi.param) and np.array_equal(m.cpu().numpy(), mi.mom)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fp32_stages_at_kernel_level(dtype):
    """The three HBM passes on their own, tighter than the step's 1e-5, over
    every kernel class (fused, 128- and 256-tile) with a warm momentum:
      K1  momentum mu M + (1 - mu) G and its norm, 1e-6 relative to fp64;
      K2  X0 (the first bf16 iterate, read from the workspace after one
          iteration) is the round-to-nearest of M / (nu + eps), taken from the
          library's own M and nu: within half a bf16 ulp of the fp64 quotient;
      K5  p (1 - lr wd) - lr s O for the library's own O, 1e-6."""
    lr, mu, wd = 0.03, 0.9, 0.05
    shapes = [(40, 300), (300, 100), (640, 200), (1100, 1030)]
    inputs = [W.adhoc_inputs(r, c, dtype, seed=900 + k, mom_std=0.5) for k, (r, c) in enumerate(shapes)]
    run = Run(inputs).step(lr=lr, mu=mu, wd=wd, ns_steps=1, rms_scale="sqrt_max1")
    for i, mi in enumerate(inputs):
        want_m = mu * mi.mom.astype(np.float64) + (1 - mu) * mi.grad.astype(np.float64)
        e_m = rel(run.mom(i), want_m)
        m_lib = run.mom(i).astype(np.float64)
        e_nu = abs(run.nu(i) - np.linalg.norm(m_lib)) / np.linalg.norm(m_lib)
        x = m_lib / (run.nu(i) + 1e-7)
        got = run.x(i, 0)[:mi.rows, :mi.cols].astype(np.float64)
        half_ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 1e-30))) - 8)
        ok_x = np.all(np.abs(got - x) <= half_ulp * (1 + 2.0 ** -12) + 1e-38)
        s = math.sqrt(max(1.0, mi.rows / mi.cols))
        e_p = check_apply_consistency(run, i, lr, wd, s, tol=1e-6)
        say(f"  {mi.rows}x{mi.cols} {dtype}: M {e_m:.1e} nu {e_nu:.1e} X0 RNE {ok_x} apply {e_p:.1e}")
        assert e_m <= 1e-6 and e_nu <= 1e-6 and ok_x
