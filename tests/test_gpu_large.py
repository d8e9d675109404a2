"""A matrix of 2^32 elements (2^20 x 4096, the longest side allowed): every
element offset past 32 bits, the tall layout, a 2^20-deep Gram contraction.
The oracle cannot run the whole matrix, so the input is built so that the
exact answer follows from a small one: G = 1_k (x) B, k = 1024 copies of a
1024 x 4096 block B stacked vertically.  Then G^T G = k B^T B, the
normalised input is the normalised B scaled by 1/sqrt(k) = 1/32 (a power of
two, so the bf16 rounding commutes with it), the Newton-Schulz iteration
keeps the block structure, and NS(G) = 1_k (x) NS(B) / 32, with NS(B) from
the fp64 oracle on B alone (the iteration acts on singular values, so the
short-side choice of the small and the large problem does not matter).
Checked on the device, block by block: momentum (1 - mu) G to 1e-6, O
against 1_k (x) NS(B) / 32 to 2e-2, and the applied update against the
library's own O to 1e-5 (s = sqrt(rows / cols) = 16)."""
import math

import numpy as np
import pytest
import torch

import matrix_aware_optimizer_libmuon_amd as muon
from matrix_aware_optimizer_libmuon_amd import workloads as W
from oracle import muon_oracle as O
from tests.gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu

K_COPIES, BR, BC = 1024, 1024, 4096


@pytest.mark.timeout(400)
def test_two_to_the_32_elements_block_repeated():
    lr, mu, wd = 0.02, 0.95, 0.01
    rows, cols = K_COPIES * BR, BC
    assert rows == 1 << 20 and rows * cols == 1 << 32
    b = W.adhoc_inputs(BR, BC, "bf16", seed=4242)
    say(f"large: {rows} x {cols} = 2^32 elements, block {BR} x {BC} repeated {K_COPIES} times")
    gb = torch.from_numpy(b.grad_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    pb = torch.from_numpy(b.param).to(DEV)
    g = gb.repeat(K_COPIES, 1)
    p = pb.repeat(K_COPIES, 1)
    m = torch.zeros(rows, cols, device=DEV)
    ws = muon.alloc_workspace([(rows, cols)], DEV)
    muon.muon_step([p], [g], [m], lr=lr, mu=mu, wd=wd, ns_steps=5, rms_scale="sqrt_max1",
                   workspace=ws)
    torch.cuda.synchronize()
    say("  step done")
    ref = O.muon_step_matrix(b.param, b.grad, np.zeros((BR, BC)), lr=lr, mu=mu, wd=wd, ns_steps=5)
    o_b = torch.from_numpy(ref["o"] / math.sqrt(K_COPIES)).to(DEV)           # fp64
    omu = torch.tensor(1.0, dtype=torch.float32) - torch.tensor(mu, dtype=torch.float32)
    m_b = gb.float() * omu.to(DEV)
    v = muon.workspace_view([(rows, cols)], 0, 5)
    assert v["rows_pad"] == rows and v["cols_pad"] == cols
    o = ws[v["o_off"]:v["o_off"] + rows * cols * 2].view(torch.bfloat16).view(K_COPIES, BR, BC)
    s = math.sqrt(rows / cols)
    decay = 1.0 - lr * wd
    num_m = num_o = num_p = den_o = den_p = 0.0
    for k0 in range(0, K_COPIES, 64):                      # 64 blocks (1 GiB of fp32) at a time
        sl = slice(k0 * BR, (k0 + 64) * BR)
        mk = m[sl].view(64, BR, BC)
        num_m = max(num_m, (mk - m_b).abs().max().item() / m_b.abs().max().item())
        ok = o[k0:k0 + 64].double()
        num_o += (ok - o_b).square().sum().item()
        den_o += 64 * o_b.square().sum().item()
        want_p = pb.double() * decay - lr * s * ok
        num_p += (p[sl].view(64, BR, BC).double() - want_p).square().sum().item()
        den_p += want_p.square().sum().item()
    e_o, e_p = math.sqrt(num_o / den_o), math.sqrt(num_p / den_p)
    say(f"  momentum max rel {num_m:.2e}, O {e_o:.3e}, apply {e_p:.2e}")
    assert num_m <= 1e-6
    assert e_o <= 2e-2
    assert e_p <= 1e-5
