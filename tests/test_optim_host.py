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


def test_torch_optim_muon_keyword_names_map_onto_the_groups():
    w = torch.nn.Parameter(torch.zeros(4, 6))
    opt = Muon([w], lr=0.01, momentum=0.9, weight_decay=0.1, ns_coefficients=(2.0, -1.5, 0.5),
               adjust_lr_fn="original", nesterov=True)
    g = opt.param_groups[0]
    assert g["wd"] == 0.1 and g["coeffs"] == (2.0, -1.5, 0.5) and g["rms_scale"] == "sqrt_max1"
    assert g["lr"] == 0.01 and g["momentum"] == 0.9 and g["nesterov"] is True
    with pytest.raises(ValueError):
        Muon([w], adjust_lr_fn="match_rms_adamw")
