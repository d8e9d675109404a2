"""The tail split of the symmetric launches against the fp64 oracle (a design
that was tried and is not in the library: its first GPU run faulted.  Its
compiled kernels formed load bases with v_readfirstlane_b32 0 wait states
before the asm loads that read them (tests/test_isa_hazards.py holds the
library to 5), so a load could take a stale base.  These tests stay skipped
while the split is out of the library).

26 matrices of the 256-tile class (13 tall 2048 x 1024, 13 wide 1024 x 2048)
have 260 upper tiles: one full wave of 256 and a tail of 4, so the last 4
tiles of the Gram and C launches are computed in parts over K (8 each here:
the Gram's K = 2048 and C's K = 1024 leave 8 steps of 32 per part) and summed
by the last part of each tile.  Both orientations (the tall matrices read X
through its MN-contiguous view), two consecutive eager steps (the per-tile
counters must be back at zero for the second), and two prepared-plan steps
under MUON_DEBUG (the partial tiles are NaN-filled first, so a part summed
before it was written would show).  The Mamba set (128-tile tail with split
C) and the single 8192 x 28672 matrix (16 parts per tile) are covered by
test_gpu_workloads.py."""
import os

import numpy as np
import pytest
import torch

import matrix_aware_optimizer_libmuon_amd as muon
from matrix_aware_optimizer_libmuon_amd import workloads as W
from oracle import muon_oracle as O
from tests.gpu_helpers import DEV, Run, check_apply_consistency, grad_tensor, rel, say

pytestmark = [pytest.mark.gpu, pytest.mark.skip(
    reason="the tail split faulted the GPU (illegal address) on its first run: its load bases "
           "were written by vector instructions 0 wait states before the loads; the split is "
           "not in the library")]

SHAPES = [(2048, 1024)] * 13 + [(1024, 2048)] * 13


def _check_step(run, inputs, state, lr, mu, wd):
    worst = 0.0
    for i, mi in enumerate(inputs):
        p_prev, m_prev = state[i]
        out = O.muon_step_matrix(p_prev, mi.grad, m_prev, lr=lr, mu=mu, wd=wd)
        e_o = rel(run.o(i), out["o"])
        worst = max(worst, e_o)
        assert rel(run.mom(i), out["m"]) <= 1e-5, i
        assert e_o <= 2e-2, (i, SHAPES[i], e_o)
        check_apply_consistency(run, i, lr, wd, 1.0)
        state[i] = (run.param(i).astype(np.float64), out["m"])
    return worst


def test_tail_split_two_steps_tall_and_wide():
    assert sum((min(r, c) // 256) * (min(r, c) // 256 + 1) // 2 for r, c in SHAPES) == 260
    inputs = [W.adhoc_inputs(r, c, "bf16", seed=1100 + k) for k, (r, c) in enumerate(SHAPES)]
    run = Run(inputs)
    state = [(mi.param.astype(np.float64), mi.mom.astype(np.float64)) for mi in inputs]
    run.step(lr=0.02, mu=0.95, wd=0.01)
    say(f"  split step 1: worst O {_check_step(run, inputs, state, 0.02, 0.95, 0.01):.3e}")
    inputs = [W.adhoc_inputs(r, c, "bf16", seed=1200 + k) for k, (r, c) in enumerate(SHAPES)]
    for i, mi in enumerate(inputs):
        mi.param = run.param(i)
    run.set_grads(inputs)
    run.step(lr=0.02, mu=0.95, wd=0.01)
    say(f"  split step 2: worst O {_check_step(run, inputs, state, 0.02, 0.95, 0.01):.3e}")


def test_tail_split_plan_steps_under_debug():
    old = os.environ.get("MUON_DEBUG")
    os.environ["MUON_DEBUG"] = "1"
    try:
        inputs = [W.adhoc_inputs(r, c, "bf16", seed=1300 + k) for k, (r, c) in enumerate(SHAPES)]
        params = [torch.from_numpy(mi.param).to(DEV) for mi in inputs]
        moms = [torch.from_numpy(mi.mom).to(DEV) for mi in inputs]
        grads = [grad_tensor(mi) for mi in inputs]
        plan = muon.Plan(params, grads, moms, lr=0.02, mu=0.95, wd=0.01)
        state = [(mi.param.astype(np.float64), mi.mom.astype(np.float64)) for mi in inputs]
        for step in range(2):
            plan.step()
            torch.cuda.synchronize()
            worst = 0.0
            for i, mi in enumerate(inputs):
                p_prev, m_prev = state[i]
                out = O.muon_step_matrix(p_prev, mi.grad, m_prev, lr=0.02, mu=0.95, wd=0.01)
                p = params[i].cpu().numpy()
                assert np.isfinite(p).all()
                e = rel(p - p_prev * (1 - 0.02 * 0.01), out["p"] - p_prev * (1 - 0.02 * 0.01))
                worst = max(worst, e)
                assert e <= 2e-2, (step, i, e)
                assert rel(moms[i].cpu().numpy(), out["m"]) <= 1e-5
                state[i] = (p.astype(np.float64), out["m"])
            say(f"  plan step {step + 1} under MUON_DEBUG: worst update error {worst:.3e}")
        del plan
    finally:
        if old is None:
            del os.environ["MUON_DEBUG"]
        else:
            os.environ["MUON_DEBUG"] = old
