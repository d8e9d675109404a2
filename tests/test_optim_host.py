"""CPU-side checks of the hybrid optimizer class: it refuses what libmuon
cannot update (no GPU needed; nothing is launched)."""
import pytest

torch = pytest.importorskip("torch")

from matrix_aware_optimizer_libmuon_amd.optim import Muon  # noqa: E402


def test_rejects_non_2d_weights_in_a_muon_group():
    with pytest.raises(ValueError):
        Muon([torch.nn.Parameter(torch.zeros(4))])
    with pytest.raises(ValueError):
        Muon([torch.nn.Parameter(torch.zeros(2, 3, 4))])


def test_rejects_non_fp32_parameters():
    with pytest.raises(ValueError):
        Muon([torch.nn.Parameter(torch.zeros(4, 4, dtype=torch.float64))])


def test_adamw_groups_take_any_shape():
    opt = Muon([{"params": [torch.nn.Parameter(torch.zeros(4, 4))]},
                {"params": [torch.nn.Parameter(torch.zeros(7)), torch.nn.Parameter(torch.zeros(2, 3, 4))],
                 "muon": False}])
    assert opt.param_groups[1]["muon"] is False and opt.param_groups[0]["lr"] == 0.02
    assert opt.param_groups[1]["adamw_lr"] == 1e-3 and opt.param_groups[1]["adamw_betas"] == (0.9, 0.95)
