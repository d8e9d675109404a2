"""GPU parity of the AdamW branch (muon_adamw_step through the C ABI) with the
fp64 oracle ("Muon meets Mamba", section 4.2, _step_adamw): four consecutive
steps over ragged tensor sizes (odd, not multiples of 8, a misaligned view
that takes the scalar path, one larger tensor), fp32 and bf16 gradients, a
tensor without a gradient; fp32 path bar: relative Frobenius error <= 1e-5 on
param, first and second moment after every step."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import matrix_aware_optimizer_libmuon_amd as muon  # noqa: E402
from matrix_aware_optimizer_libmuon_amd import workloads as W  # noqa: E402
import oracle  # noqa: E402
from tests.gpu_helpers import DEV, rel, say  # noqa: E402

pytestmark = pytest.mark.gpu

SIZES = [1, 7, 8, 129, 1000, 4096, 3 * 5 * 7 * 11, 16384 + 3, 1 << 20]
LR, BETAS, EPS, WD = 1e-3, (0.9, 0.95), 1e-8, 0.01
STEPS = 4
TOL = 1e-5


def _grad_tensor(inp, t, dtype):
    if dtype == "bf16":
        return torch.from_numpy(inp.grad_bits[t].view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(inp.grads[t]).to(DEV)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_adamw_matches_oracle_over_steps(dtype):
    inputs = [W.adamw_inputs(n, STEPS, dtype, seed=i, warm=(i % 3 == 1)) for i, n in enumerate(SIZES)]
    skip = 2  # tensor 2 never has a gradient
    # a misaligned view: the last tensor lives at offset 1 of a larger buffer
    store = []
    p, m, v = [], [], []
    for i, inp in enumerate(inputs):
        if i == len(inputs) - 1:
            big = torch.zeros(3, inp.numel + 1, dtype=torch.float32, device=DEV)
            big[0, 1:] = torch.from_numpy(inp.param).to(DEV)
            big[1, 1:] = torch.from_numpy(inp.exp_avg).to(DEV)
            big[2, 1:] = torch.from_numpy(inp.exp_avg_sq).to(DEV)
            store.append(big)
            p.append(big[0, 1:]); m.append(big[1, 1:]); v.append(big[2, 1:])
        else:
            p.append(torch.from_numpy(inp.param).to(DEV))
            m.append(torch.from_numpy(inp.exp_avg).to(DEV))
            v.append(torch.from_numpy(inp.exp_avg_sq).to(DEV))
    ref = [(inp.param.astype(np.float64), inp.exp_avg.astype(np.float64), inp.exp_avg_sq.astype(np.float64))
           for inp in inputs]
    counts = [0] * len(inputs)
    ws = muon.alloc_adamw_workspace(len(inputs), DEV)
    worst = 0.0
    for t in range(STEPS):
        grads = [None if i == skip else _grad_tensor(inp, t, dtype) for i, inp in enumerate(inputs)]
        for i in range(len(inputs)):
            if grads[i] is not None:
                counts[i] += 1
        muon.adamw_step(p, grads, m, v, [max(c, 1) for c in counts], lr=LR, betas=BETAS, eps=EPS, wd=WD,
                        workspace=ws)
        torch.cuda.synchronize()
        for i, inp in enumerate(inputs):
            if i == skip:
                continue
            ref[i] = oracle.adamw_step_tensor(*ref[i][:1], inp.grads[t], ref[i][1], ref[i][2], counts[i],
                                              lr=LR, betas=BETAS, eps=EPS, wd=WD)
            for name, dev, want in (("p", p[i], ref[i][0]), ("m", m[i], ref[i][1]), ("v", v[i], ref[i][2])):
                err = rel(dev.cpu().numpy(), want)
                worst = max(worst, err)
                assert err <= TOL, f"step {t + 1} tensor {i} (numel {inp.numel}) {name}: {err}"
    # the tensor without a gradient is untouched
    assert np.array_equal(p[skip].cpu().numpy(), inputs[skip].param)
    assert np.array_equal(m[skip].cpu().numpy(), inputs[skip].exp_avg)
    say(f"adamw {dtype}: worst relative error over {STEPS} steps {worst:.3g}")


def test_adamw_grouped_equals_one_by_one():
    inputs = [W.adamw_inputs(n, 1, "bf16", seed=50 + i) for i, n in enumerate(SIZES)]
    runs = []
    for grouped in (True, False):
        p = [torch.from_numpy(x.param).to(DEV) for x in inputs]
        m = [torch.from_numpy(x.exp_avg).to(DEV) for x in inputs]
        v = [torch.from_numpy(x.exp_avg_sq).to(DEV) for x in inputs]
        g = [_grad_tensor(x, 0, "bf16") for x in inputs]
        if grouped:
            muon.adamw_step(p, g, m, v, [1] * len(p))
        else:
            for k in range(len(p)):
                muon.adamw_step([p[k]], [g[k]], [m[k]], [v[k]], [1])
        torch.cuda.synchronize()
        runs.append([t.cpu().numpy() for t in p + m + v])
    for a, b in zip(*runs):
        assert np.array_equal(a, b)
