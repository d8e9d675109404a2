"""The seeded input generator: determinism, shapes, distributions, and the
bf16 rounding of inputs checked against torch's own float32 -> bfloat16
conversion (round to nearest even)."""
import numpy as np
import torch

from matrix_aware_optimizer_libmuon_amd import workloads as W


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 10.0 ** r.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 3.0e38, 1e-40],
                                 dtype=np.float32)]).astype(np.float32)
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(W.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_ties_round_to_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties to even -> 1
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], dtype=np.float32)
    assert list(W.round_to_bf16(x)) == [1.0, 1.0 + 2 * 2.0 ** -7]


def test_shapes():
    assert W.WORKLOADS[1].shapes == ((256, 768),)
    w2 = W.WORKLOADS[2]
    assert w2.n_mats == 96 and w2.shapes[:4] == ((768, 3072), (1536, 80), (48, 1536), (1536, 768))
    w3 = W.WORKLOADS[3]
    assert w3.n_mats == 224 and w3.elements() == 32 * (4 * 4096 ** 2 + 3 * 4096 * 14336)
    w4 = W.WORKLOADS[4]
    assert w4.n_mats == 2048
    rs = {r for r, _ in w4.shapes}
    cs = {c for _, c in w4.shapes}
    assert rs == cs == {64, 128, 256, 512}
    assert any(r > c for r, c in w4.shapes) and any(r < c for r, c in w4.shapes)
    assert W.WORKLOADS[5].shapes == ((8192, 28672),)
    assert W.layer_subset(w3, [0, 31])[-1] == 223


def test_nominal_flops():
    # 5 * (4 m^2 n + 2 m^3) for the single 256 x 768 gradient
    assert W.WORKLOADS[1].ns_flops() == 5 * (4 * 256 * 256 * 768 + 2 * 256 ** 3)
    assert abs(W.WORKLOADS[3].ns_flops() / 1e12 - 791.6) < 0.1


def test_determinism_and_independence():
    w = W.WORKLOADS[2]
    a = W.matrix_inputs(w, 5, step=1)
    b = W.matrix_inputs(w, 5, step=1)
    assert np.array_equal(a.grad_bits, b.grad_bits) and np.array_equal(a.param, b.param)
    c = W.matrix_inputs(w, 5, step=2)
    assert not np.array_equal(a.grad_bits, c.grad_bits)
    assert np.array_equal(a.param, c.param)            # params are drawn once
    got = dict(W.iter_inputs(w, indices=[7, 5, 9], step=1, threads=3))
    assert np.array_equal(got[5].grad_bits, a.grad_bits)


def test_distributions():
    w1 = W.WORKLOADS[1]
    g, bits = W.grad(w1, 0, 0)
    assert bits is None and g.dtype == np.float32 and abs(g.std() - 1) < 0.01
    w2 = W.WORKLOADS[2]
    g, bits = W.grad(w2, 0, 0)
    assert bits.dtype == np.uint16 and abs(g.std() - 0.02) < 0.0005
    assert np.array_equal(W.round_to_bf16(g), g)
    assert np.all(W.momentum(w2, 0) == 0)
    p = W.param(w2, 0)
    assert abs(p.std() - 0.02) < 0.0005


def test_spiked_gradient_is_ill_conditioned():
    # a small stand-in of the transformer workload's rank-8 spike: top
    # singular values far above the bulk
    w = W.Workload(3, "spike test", ((256, 512),), "bf16", 1)
    g, _ = W.grad(w, 0, 0)
    s = np.linalg.svd(g.astype(np.float64), compute_uv=False)
    assert s[0] / s[8] > 5 and s[7] / s[8] > 5
