"""The oracle's whole step against an independent library implementation of
the same method: PyTorch's own ``torch.optim.Muon`` (run on the CPU, as a
black box, from its documented semantics: EMA momentum buffer, the optional
look-ahead input ``grad.lerp(buf, momentum)``, the quintic iteration on the
short side of the Frobenius-normalised input, decoupled weight decay, and the
update scaled by sqrt(max(1, rows / cols)) under ``adjust_lr_fn="original"``).
These are the readings the oracle takes from the pages, so the two must agree
step after step, with the momentum carried:

* momentum buffer: 1e-6 relative (fp32 against fp64);
* orthogonalised matrix O, recovered from the parameter change: 3e-2
  relative -- PyTorch runs the iteration entirely in bf16 (each of A,
  b A + c A^2 and the new X rounded to bf16, five times over), the oracle in
  fp64; the observed gap is 1.1-2.0e-2;
* parameter: follows from the two above.

Planted mistakes in the oracle (monkeypatched copies, CPU only) must each
break the agreement.  The library implementation is not involved."""
import numpy as np
import pytest
import torch

from oracle import muon_oracle as O

LR, MU, WD = 0.02, 0.95, 0.01
SHAPES = [(64, 96), (96, 64), (80, 80), (33, 150), (150, 33), (256, 768)]

pytestmark = pytest.mark.skipif(not hasattr(torch.optim, "Muon"), reason="torch.optim.Muon missing")


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _compare(shape, nesterov, seed, steps=2):
    """Worst (momentum, O) relative differences over `steps` steps."""
    rng = np.random.default_rng(seed)
    r, c = shape
    p0 = (rng.standard_normal((r, c)) * 0.02).astype(np.float32)
    p = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.Muon([p], lr=LR, weight_decay=WD, momentum=MU, nesterov=nesterov,
                           adjust_lr_fn="original")
    m = np.zeros((r, c))
    worst_m = worst_o = 0.0
    for _ in range(steps):
        g = rng.standard_normal((r, c)).astype(np.float32)
        before = p.detach().numpy().astype(np.float64).copy()
        p.grad = torch.from_numpy(g)
        opt.step()
        ref = O.muon_step_matrix(before, g, m, lr=LR, mu=MU, wd=WD, rms_mode="sqrt_max1",
                                 nesterov=nesterov)
        m = ref["m"]
        buf = opt.state[p]["momentum_buffer"].numpy().astype(np.float64)
        after = p.detach().numpy().astype(np.float64)
        o_torch = (before * (1 - LR * WD) - after) / (LR * ref["scale"])
        worst_m = max(worst_m, _rel(buf, ref["m"]))
        worst_o = max(worst_o, _rel(o_torch, ref["o"]))
    return worst_m, worst_o


@pytest.mark.parametrize("nesterov", [False, True])
@pytest.mark.parametrize("shape", SHAPES)
def test_oracle_step_agrees_with_torch_muon(shape, nesterov):
    e_m, e_o = _compare(shape, nesterov, seed=sum(shape) + nesterov)
    assert e_m <= 1e-6, e_m
    assert e_o <= 3e-2, e_o


def _plant(monkeypatch, mistake):
    if mistake == "momentum_sum":                  # M + G instead of the EMA
        monkeypatch.setattr(O, "momentum_lerp", lambda m, g, mu: mu * O.as_f64(m) + O.as_f64(g))
    elif mistake == "scale_inverted":              # sqrt(max(1, cols / rows))
        monkeypatch.setattr(O, "rms_scale", lambda r, c, mode: float(np.sqrt(max(1.0, c / r))))
    elif mistake == "flip_b":                      # wrong sign of the linear coefficient
        ns = O.newton_schulz
        monkeypatch.setattr(O, "newton_schulz", lambda g, coeffs, steps, eps:
                            ns(g, tuple((a, -b, c) for a, b, c in coeffs), steps, eps))
    elif mistake == "nesterov_wrong_pull":         # mu G + (1 - mu) M
        monkeypatch.setattr(O, "nesterov_input",
                            lambda m, g, mu: mu * O.as_f64(g) + (1 - mu) * O.as_f64(m))


@pytest.mark.parametrize("mistake", ["momentum_sum", "scale_inverted", "flip_b", "nesterov_wrong_pull"])
def test_planted_oracle_mistakes_break_the_agreement(monkeypatch, mistake):
    _plant(monkeypatch, mistake)
    caught = False
    for shape in [(96, 64), (64, 96)]:
        e_m, e_o = _compare(shape, nesterov=True, seed=5)
        caught |= e_m > 1e-6 or e_o > 3e-2
    assert caught, mistake
