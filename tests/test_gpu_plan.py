"""The prepared step (muon_plan_create / muon_plan_step): equal to muon_step,
and capturable in a CUDA (HIP) graph whose replays, with eager work and
synchronisations between them and a learning-rate schedule written into the
device hyper-parameters, match an eager plan step by step."""
import numpy as np
import pytest
import torch

import matrix_aware_optimizer_libmuon_amd as muon
from matrix_aware_optimizer_libmuon_amd import workloads as W
from tests.gpu_helpers import DEV, grad_tensor, rel, say

pytestmark = pytest.mark.gpu

# one per kernel class: fused (small), 128-tile, 256-tile; wide and tall
SHAPES = [(48, 200), (200, 48), (300, 520), (1100, 1030)]


def _state(seed):
    inputs = [W.adhoc_inputs(r, c, "bf16", seed=seed + k, mom_std=0.2) for k, (r, c) in enumerate(SHAPES)]
    p = [torch.from_numpy(mi.param).to(DEV) for mi in inputs]
    m = [torch.from_numpy(mi.mom).to(DEV) for mi in inputs]
    g = [grad_tensor(mi) for mi in inputs]
    return inputs, p, g, m


def test_plan_step_equals_muon_step():
    _, p1, g1, m1 = _state(1000)
    _, p2, g2, m2 = _state(1000)
    plan = muon.Plan(p2, g2, m2, lr=0.02, mu=0.9, wd=0.01, ns_steps=5)
    for _ in range(2):
        muon.muon_step(p1, g1, m1, lr=0.02, mu=0.9, wd=0.01, ns_steps=5)
        plan.step()
    torch.cuda.synchronize()
    for a, b, c, d in zip(p1, p2, m1, m2):
        # equal up to the order of the fp64 atomic norm accumulation
        assert rel(a.cpu().numpy(), b.cpu().numpy()) <= 1e-6
        assert np.array_equal(c.cpu().numpy(), d.cpu().numpy())
    plan.close()


@pytest.mark.parametrize("variant", [{}, {"zero_centering": True, "ns_first": True}])
def test_plan_replays_in_a_graph(variant):
    _, pe, ge, me = _state(2000)      # eager plan
    _, pg, gg, mg = _state(2000)      # captured plan, same start
    lrs = [0.02, 0.01, 0.005]
    eager = muon.Plan(pe, ge, me, lr=lrs[0], mu=0.9, wd=0.05, ns_steps=5, **variant)
    graphed = muon.Plan(pg, gg, mg, lr=lrs[0], mu=0.9, wd=0.05, ns_steps=5, **variant)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        graph.capture_begin()
        graphed.step()
        graph.capture_end()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for t, lr in enumerate(lrs):
        # new gradients written into the same buffers (eager work between replays)
        for k, (a, b) in enumerate(zip(ge, gg)):
            new = torch.randn(a.shape, generator=torch.Generator(device=DEV).manual_seed(31 * t + k),
                              device=DEV).to(a.dtype)
            a.copy_(new)
            b.copy_(new)
        eager.set_hyper(lr=lr)
        graphed.set_hyper(lr=lr)
        eager.step()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        worst = 0.0
        for a, b, c, d in zip(pe, pg, me, mg):
            worst = max(worst, rel(a.cpu().numpy(), b.cpu().numpy()), rel(c.cpu().numpy(), d.cpu().numpy()))
        say(f"  replay {t} (lr {lr}): worst relative difference to the eager step {worst:.2e}")
        assert worst <= 1e-6
    eager.close()
    graphed.close()
