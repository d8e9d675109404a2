"""The hybrid optimizer class (Muon groups + AdamW groups, the interface of
"Muon meets Mamba", sections 4.1-4.3) against the fp64 oracles: two steps of
a small parameter set with 2-D hidden weights (wide and tall), a 1-D bias and
an embedding-like matrix in an AdamW group."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from matrix_aware_optimizer_libmuon_amd import workloads as W  # noqa: E402
from matrix_aware_optimizer_libmuon_amd.optim import Muon  # noqa: E402
import oracle  # noqa: E402
from tests.gpu_helpers import DEV, rel  # noqa: E402

pytestmark = pytest.mark.gpu


def test_hybrid_optimizer_two_steps_match_oracles():
    lr, mu, wd = 0.02, 0.95, 0.01
    hidden_shapes = [(256, 768), (768, 256)]
    other_sizes = [768, 1000 * 64]
    hid = [W.adhoc_inputs(r, c, "bf16", seed=300 + i) for i, (r, c) in enumerate(hidden_shapes)]
    oth = [W.adamw_inputs(n, 2, "bf16", seed=400 + i) for i, n in enumerate(other_sizes)]
    ph = [torch.nn.Parameter(torch.from_numpy(h.param).to(DEV)) for h in hid]
    po = [torch.nn.Parameter(torch.from_numpy(o.param).to(DEV)) for o in oth]
    opt = Muon([{"params": ph}, {"params": po, "muon": False}])
    ref_o = [(o.param.astype(np.float64), np.zeros(o.numel), np.zeros(o.numel)) for o in oth]
    for t in range(2):
        g_hid = [h.grad if t == 0 else W.adhoc_inputs(h.rows, h.cols, "bf16", seed=500 + 10 * k + t).grad
                 for k, h in enumerate(hid)]
        for p, g in zip(ph, g_hid):
            p.grad = torch.from_numpy(g).to(DEV)  # fp32 holding bf16-exact values
        for p, o in zip(po, oth):
            p.grad = torch.from_numpy(o.grads[t]).to(DEV)
        p_before = [p.detach().cpu().numpy().astype(np.float64) for p in ph]
        m_before = [np.zeros(p.shape) if t == 0 else opt.state[p]["momentum_buffer"].cpu().numpy()
                    for p in ph]
        opt.step()
        torch.cuda.synchronize()
        for k, p in enumerate(ph):
            out = oracle.muon_step_matrix(p_before[k], g_hid[k], m_before[k], lr=lr, mu=mu, wd=wd,
                                          ns_steps=5)
            assert rel(opt.state[p]["momentum_buffer"].cpu().numpy(), out["m"]) <= 1e-5
            got = p.detach().cpu().numpy() - p_before[k] * (1.0 - lr * wd)
            assert rel(got, -lr * out["o"]) <= 2e-2
        for k, (p, o) in enumerate(zip(po, oth)):
            ref_o[k] = oracle.adamw_step_tensor(ref_o[k][0], o.grads[t], ref_o[k][1], ref_o[k][2], t + 1)
            assert rel(p.detach().cpu().numpy(), ref_o[k][0]) <= 1e-5
            assert rel(opt.state[p]["exp_avg"].cpu().numpy(), ref_o[k][1]) <= 1e-5
            assert opt.state[p]["step"] == t + 1


def test_muon_groups_take_only_2d_weights():
    with pytest.raises(ValueError):
        Muon([torch.nn.Parameter(torch.zeros(4, device=DEV))])


@pytest.mark.parametrize("variant", [dict(zero_centering=True, nesterov=True),
                                     dict(zero_centering=True, ns_first=True)])
def test_optimizer_group_variants_match_oracle(variant):
    lr, mu, wd = 0.02, 0.95, 0.01
    hid = [W.adhoc_inputs(r, c, "f32", seed=600 + i, col_offset=0.5)
           for i, (r, c) in enumerate([(192, 320), (320, 192)])]
    ph = [torch.nn.Parameter(torch.from_numpy(h.param).to(DEV)) for h in hid]
    opt = Muon([dict(params=ph, **variant)])
    for p, h in zip(ph, hid):
        p.grad = torch.from_numpy(h.grad).to(DEV)
    opt.step()
    torch.cuda.synchronize()
    for p, h in zip(ph, hid):
        out = oracle.muon_step_matrix(h.param, h.grad, np.zeros((h.rows, h.cols)), lr=lr, mu=mu,
                                      wd=wd, ns_steps=5, **variant)
        m = opt.state[p]["momentum_buffer"].cpu().numpy()
        assert rel(m, out["m"]) <= (2e-2 if variant.get("ns_first") else 1e-5)
        got = p.detach().cpu().numpy() - h.param.astype(np.float64) * (1.0 - lr * wd)
        want = out["p"] - h.param.astype(np.float64) * (1.0 - lr * wd)
        assert rel(got, want) <= 2e-2


@pytest.mark.skipif(not hasattr(torch.optim, "Muon"), reason="torch.optim.Muon missing")
def test_drop_in_for_torch_optim_muon():
    """The same two steps through this optimizer (on the GPU) and through
    PyTorch's ``torch.optim.Muon`` (on the CPU), constructed with PyTorch's
    keyword names: momentum buffers to 1e-5; the orthogonalised update to
    4e-2 (each side is within 2e-2 of the exact step: bf16 iterations with
    fp32 accumulation here, all-bf16 arithmetic in PyTorch's)."""
    kw = dict(lr=0.02, momentum=0.95, weight_decay=0.01, nesterov=True, adjust_lr_fn="original")
    shapes = [(256, 768), (768, 256), (1100, 1030)]
    rng = np.random.default_rng(77)
    p0 = [(rng.standard_normal(s) * 0.02).astype(np.float32) for s in shapes]
    ours = [torch.nn.Parameter(torch.from_numpy(p).to(DEV)) for p in p0]
    ref = [torch.nn.Parameter(torch.from_numpy(p.copy())) for p in p0]
    opt_ours, opt_ref = Muon(ours, **kw), torch.optim.Muon(ref, **kw)
    for _ in range(2):
        before_a = [p.detach().cpu().numpy().astype(np.float64) for p in ours]
        before_b = [p.detach().numpy().astype(np.float64) for p in ref]
        for a, b, s in zip(ours, ref, shapes):
            g = rng.standard_normal(s).astype(np.float32)
            a.grad = torch.from_numpy(g).to(DEV)
            b.grad = torch.from_numpy(g)
        opt_ours.step()
        opt_ref.step()
        torch.cuda.synchronize()
        for a, b, pa, pb in zip(ours, ref, before_a, before_b):
            ma = opt_ours.state[a]["momentum_buffer"].cpu().numpy()
            mb = opt_ref.state[b]["momentum_buffer"].numpy()
            assert rel(ma, mb) <= 1e-5
            da = a.detach().cpu().numpy() - pa * (1 - 0.02 * 0.01)
            db = b.detach().numpy() - pb * (1 - 0.02 * 0.01)
            assert rel(da, db) <= 4e-2
