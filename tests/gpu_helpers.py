"""Helpers of the GPU tests: move seeded inputs to the device, run the library
through its C ABI binding, and read every stage back (momentum, norm, the
final bf16 iterate O from the workspace, the new parameter)."""
import sys

import numpy as np
import torch

import matrix_aware_optimizer_libmuon_amd as muon
from matrix_aware_optimizer_libmuon_amd import workloads as W

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


def grad_tensor(mi: W.MatrixInputs):
    if mi.grad_bits is not None:
        return torch.from_numpy(mi.grad_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(mi.grad).to(DEV)


def bf16_to_np(t):
    return t.float().cpu().numpy()


class Run:
    """One muon_step over a list of MatrixInputs; keeps device tensors."""

    def __init__(self, inputs, grads_present=None):
        self.inputs = inputs
        self.shapes = [(mi.rows, mi.cols) for mi in inputs]
        self.p = [torch.from_numpy(mi.param).to(DEV) for mi in inputs]
        self.m = [torch.from_numpy(mi.mom).to(DEV) for mi in inputs]
        self.g = [grad_tensor(mi) if (grads_present is None or grads_present[i]) else None
                  for i, mi in enumerate(inputs)]
        self.ws = muon.alloc_workspace(self.shapes, DEV)
        self.p_before = None
        self.ns_steps = None

    def step(self, **kw):
        self.p_before = [t.clone() for t in self.p]
        self.ns_steps = kw.get("ns_steps", 5)
        muon.muon_step(self.p, self.g, self.m, workspace=self.ws, **kw)
        torch.cuda.synchronize()
        return self

    def set_grads(self, inputs):
        for i, mi in enumerate(inputs):
            self.g[i] = grad_tensor(mi)

    # --- read back ----------------------------------------------------------
    def ws_bf16(self, off, rows_pad, cols_pad):
        n = rows_pad * cols_pad * 2
        return self.ws[off:off + n].view(torch.bfloat16).view(rows_pad, cols_pad)

    def view(self, i, ns_steps=None):
        return muon.workspace_view(self.shapes, i, self.ns_steps if ns_steps is None else ns_steps)

    def o(self, i):
        v = self.view(i)
        r, c = self.shapes[i]
        return bf16_to_np(self.ws_bf16(v["o_off"], v["rows_pad"], v["cols_pad"]))[:r, :c]

    def x(self, i, k):
        v = self.view(i)
        return bf16_to_np(self.ws_bf16(v["x_off"][k], v["rows_pad"], v["cols_pad"]))

    def a(self, i):
        v = self.view(i)
        return bf16_to_np(self.ws_bf16(v["a_off"], v["m_pad"], v["m_pad"]))

    def c(self, i):
        """C = a I + b A + c A A (bf16 high part) of the last iteration."""
        v = self.view(i)
        return bf16_to_np(self.ws_bf16(v["c_off"], v["m_pad"], v["m_pad"]))

    def c_lo(self, i):
        """Low part of C (short side <= 128), else None."""
        v = self.view(i)
        if v["c_lo_off"] == 0:
            return None
        return bf16_to_np(self.ws_bf16(v["c_lo_off"], v["m_pad"], v["m_pad"]))

    def nu(self, i):
        off = self.view(i)["nrm2_off"]
        return float(np.sqrt(self.ws[off:off + 8].view(torch.float64).cpu().numpy()[0]))

    def mom(self, i):
        return self.m[i].cpu().numpy()

    def param(self, i):
        return self.p[i].cpu().numpy()

    def param_before(self, i):
        return self.p_before[i].cpu().numpy()


def check_apply_consistency(run, i, lr, wd, scale, tol=1e-5):
    """The new parameter equals p (1 - lr wd) - lr s O for the library's own
    O, to fp32 rounding (a property of the outputs, relating stages)."""
    p0 = run.param_before(i).astype(np.float64)
    o = run.o(i).astype(np.float64)
    want = p0 * (1.0 - lr * wd) - lr * scale * o
    err = rel(run.param(i), want)
    assert err <= tol, f"apply consistency {err}"
    return err
