"""Stream behaviour of a step whose matrices fall into both the fused class
and a tiled class: the library then runs the fused launches on a side stream
of its own, ordered after the caller's normalisation pass and before the
caller's apply pass.  Checked here: a caller stream other than the default
one, two host threads stepping at once on two streams (they share the
library's per-device side stream), and the phase-timing mode (which keeps
every launch on the caller's stream) all give the result of a plain serial
step.  Results agree to the order of the fp64 atomic norm accumulation."""
import threading

import numpy as np
import pytest
import torch

import matrix_aware_optimizer_libmuon_amd as muon
from matrix_aware_optimizer_libmuon_amd import workloads as W
from tests.gpu_helpers import DEV, grad_tensor, rel, say

pytestmark = pytest.mark.gpu

# fused (padded short side 32, 64, 128) beside 128- and 256-tile matrices
SHAPES = [(20, 300), (64, 64), (300, 100), (128, 1000), (300, 520), (1100, 1030), (33, 40)]
KW = dict(lr=0.02, mu=0.9, wd=0.01, ns_steps=5)


def _state(seed):
    inputs = [W.adhoc_inputs(r, c, "bf16", seed=seed + k, mom_std=0.2) for k, (r, c) in enumerate(SHAPES)]
    p = [torch.from_numpy(mi.param).to(DEV) for mi in inputs]
    m = [torch.from_numpy(mi.mom).to(DEV) for mi in inputs]
    g = [grad_tensor(mi) for mi in inputs]
    ws = muon.alloc_workspace(SHAPES, DEV)
    return p, g, m, ws


def _same(a_list, b_list, what):
    worst = max(rel(a.cpu().numpy(), b.cpu().numpy()) for a, b in zip(a_list, b_list))
    say(f"  {what}: worst relative difference {worst:.2e}")
    assert worst <= 1e-6, what


def _serial(seed, steps):
    p, g, m, ws = _state(seed)
    for _ in range(steps):
        muon.muon_step(p, g, m, workspace=ws, **KW)
    torch.cuda.synchronize()
    return p, m


def test_non_default_caller_stream():
    p0, m0 = _serial(500, 2)
    p, g, m, ws = _state(500)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            muon.muon_step(p, g, m, workspace=ws, stream=s, **KW)
        # read back on the caller's stream right after the step: ordered
        # after the fused launches through the join
        p_copy = [t.clone() for t in p]
    torch.cuda.synchronize()
    _same(p0, p_copy, "params, side caller stream")
    _same(m0, m, "momenta, side caller stream")


def test_two_threads_at_once():
    steps = 3
    want = [_serial(600 + 100 * k, steps) for k in range(2)]
    states = [_state(600 + 100 * k) for k in range(2)]
    streams = [torch.cuda.Stream() for _ in range(2)]
    torch.cuda.synchronize()
    errors = []

    def work(k):
        try:
            p, g, m, ws = states[k]
            with torch.cuda.stream(streams[k]):
                for _ in range(steps):
                    muon.muon_step(p, g, m, workspace=ws, stream=streams[k], **KW)
            streams[k].synchronize()
        except Exception as e:  # reported on the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k in range(2):
        _same(want[k][0], states[k][0], f"params, thread {k}")
        _same(want[k][1], states[k][2], f"momenta, thread {k}")


def test_phase_timing_mode_gives_the_same_step():
    p0, m0 = _serial(700, 2)
    p, g, m, ws = _state(700)
    muon.timing_enable(True)
    try:
        muon.timing_read()
        for _ in range(2):
            muon.muon_step(p, g, m, workspace=ws, **KW)
        torch.cuda.synchronize()
        t = muon.timing_read()
    finally:
        muon.timing_enable(False)
    assert t["ns_fused"]["launches"] >= 2 and t["x_update"]["launches"] >= 10
    _same(p0, p, "params, timing mode")
    _same(m0, m, "momenta, timing mode")
    assert np.isfinite(sum(x.sum().item() for x in p))
