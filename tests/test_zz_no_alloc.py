"""muon_step_noalloc (the step for callers that cannot allocate) against
muon_step, through the C ABI: two calls in a row on the library's fixed
scratch, the second over a smaller list, each compared with muon_step on
copies of the same inputs (momentum and parameters to 1e-5, the update
-lr*s*O to 2e-2, the tolerances of the fp32 and bf16 paths); a list whose
workspace exceeds the scratch is refused before anything changes."""
import numpy as np
import pytest
import torch

import matrix_aware_optimizer_libmuon_amd as muon
from matrix_aware_optimizer_libmuon_amd import workloads as W
from tests.gpu_helpers import DEV, grad_tensor, rel, say

pytestmark = pytest.mark.gpu

LR, MU, WD = 0.02, 0.95, 0.01


def _tensors(inputs):
    p = [torch.from_numpy(mi.param).to(DEV) for mi in inputs]
    m = [torch.from_numpy(mi.mom).to(DEV) for mi in inputs]
    g = [grad_tensor(mi) for mi in inputs]
    return p, g, m


def _compare(shapes, seed):
    inputs = [W.adhoc_inputs(r, c, "bf16", seed=seed + k, mom_std=0.01)
              for k, (r, c) in enumerate(shapes)]
    assert muon.workspace_bytes(shapes) <= muon.NOALLOC_SCRATCH_BYTES
    p_ref, g_ref, m_ref = _tensors(inputs)
    p_new, g_new, m_new = _tensors(inputs)
    muon.muon_step(p_ref, g_ref, m_ref, lr=LR, mu=MU, wd=WD, rms_scale="sqrt_max1")
    muon.muon_step_noalloc(p_new, g_new, m_new, lr=LR, mu=MU, wd=WD, rms_scale="sqrt_max1")
    torch.cuda.synchronize()
    for i, mi in enumerate(inputs):
        decayed = mi.param.astype(np.float64) * (1 - LR * WD)
        e_m = rel(m_new[i].cpu().numpy(), m_ref[i].cpu().numpy())
        e_p = rel(p_new[i].cpu().numpy(), p_ref[i].cpu().numpy())
        e_u = rel(p_new[i].cpu().numpy() - decayed, p_ref[i].cpu().numpy() - decayed)
        say(f"  noalloc {shapes[i]}: momentum {e_m:.1e} param {e_p:.1e} update {e_u:.1e}")
        assert e_m <= 1e-5 and e_p <= 1e-5 and e_u <= 2e-2, (shapes[i], e_m, e_p, e_u)


def test_noalloc_matches_muon_step_twice_then_smaller():
    # every kernel class: fused, 128-tile (wide, tall with split C), 256-tile
    _compare([(40, 300), (300, 200), (1536, 80), (1030, 1280), (96, 1000)], seed=900)
    # a second call over a smaller list reuses the same scratch
    _compare([(64, 64), (200, 130)], seed=950)


def test_noalloc_refuses_lists_beyond_the_scratch():
    shapes = [(4096, 4096)]
    assert muon.workspace_bytes(shapes) > muon.NOALLOC_SCRATCH_BYTES
    mi = W.adhoc_inputs(4096, 4096, "bf16", seed=990)
    p, g, m = _tensors([mi])
    p0 = p[0].clone()
    with pytest.raises(muon.LibMuonError) as err:
        muon.muon_step_noalloc(p, g, m, lr=LR, mu=MU, wd=WD)
    assert err.value.status == muon.MUON_EWORKSPACE
    torch.cuda.synchronize()
    assert torch.equal(p[0], p0) and not bool(m[0].any())
