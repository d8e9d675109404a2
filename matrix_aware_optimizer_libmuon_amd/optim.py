"""A torch.optim.Optimizer over libmuon: the hybrid Muon + AdamW optimizer the
pages describe, as thin marshalling around the two C calls.

Interface of the optimizer class in "Muon meets Mamba" (wmrh.cn), sections
4.1-4.3: parameter groups carry a ``muon`` flag (default True); Muon groups
take 2-D hidden-layer weights, the others (1-D biases and norm weights,
embeddings, heads) get the AdamW update with its own learning rate; weight
decay is shared.  The step variants (zero-centering of section 2.1, the
look-ahead input, the Newton-Schulz-first order) are per-group switches.
Each step issues one grouped ``muon_step`` per Muon group and one grouped
``muon_adamw_step`` per AdamW group; every per-element and per-matrix
computation runs in libmuon.so.

    opt = Muon([{"params": hidden_2d},
                {"params": others, "muon": False}])
    loss.backward(); opt.step(); opt.zero_grad()

For code written against PyTorch's own ``torch.optim.Muon`` the constructor
also takes its keyword names: ``weight_decay`` (= ``wd``), ``ns_coefficients``
(= ``coeffs``) and ``adjust_lr_fn="original"`` (= ``rms_scale="sqrt_max1"``,
the update scaled by sqrt(max(1, rows / cols))); its other scaling,
"match_rms_adamw", is not one the pages give and is refused.  The momentum
state keeps PyTorch's name, ``momentum_buffer``.  (``nesterov`` defaults to
False here, the pages' plain step; PyTorch defaults to True.)
"""
from __future__ import annotations

import torch

from . import QUINTIC, adamw_step, alloc_adamw_workspace, alloc_workspace, muon_step


class Muon(torch.optim.Optimizer):
    def __init__(self, params, lr: float = 0.02, momentum: float = 0.95, ns_steps: int = 5,
                 adamw_lr: float = 1e-3, adamw_betas=(0.9, 0.95), adamw_eps: float = 1e-8,
                 wd: float = 0.01, coeffs=QUINTIC, rms_scale: str | None = None, eps: float = 1e-7,
                 zero_centering: bool = False, nesterov: bool = False, ns_first: bool = False,
                 weight_decay: float | None = None, ns_coefficients=None,
                 adjust_lr_fn: str | None = None):
        if weight_decay is not None:
            wd = weight_decay
        if ns_coefficients is not None:
            coeffs = tuple(ns_coefficients)
        if adjust_lr_fn is not None:
            if adjust_lr_fn != "original":
                raise ValueError(f"adjust_lr_fn={adjust_lr_fn!r} is not supported; 'original' scales "
                                 "the update by sqrt(max(1, rows / cols))")
            rms_scale = "sqrt_max1"
        defaults = dict(lr=lr, momentum=momentum, ns_steps=ns_steps, adamw_lr=adamw_lr,
                        adamw_betas=tuple(adamw_betas), adamw_eps=adamw_eps, wd=wd, coeffs=coeffs,
                        rms_scale=rms_scale, eps=eps, zero_centering=zero_centering,
                        nesterov=nesterov, ns_first=ns_first, muon=True)
        super().__init__(params, defaults)
        for group in self.param_groups:
            for p in group["params"]:
                if p.dtype != torch.float32:
                    raise ValueError("libmuon updates fp32 parameters")
                if group["muon"] and p.dim() != 2:
                    raise ValueError("Muon groups take 2-D weights; put other parameters in a group "
                                     "with muon=False (AdamW)")
        self._ws = {}

    def _workspace(self, key, make):
        ws = self._ws.get(key)
        if ws is None:
            ws = self._ws[key] = make()
        return ws

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        for gi, group in enumerate(self.param_groups):
            if group["muon"]:
                self._step_muon(gi, group)
            else:
                self._step_adamw(gi, group)
        return loss

    def _step_muon(self, gi, group):
        params = [p for p in group["params"] if p.grad is not None]
        if not params:
            return
        moms = []
        for p in params:
            st = self.state[p]
            if "momentum_buffer" not in st:
                st["momentum_buffer"] = torch.zeros_like(p)
            moms.append(st["momentum_buffer"])
        shapes = tuple(tuple(p.shape) for p in params)
        ws = self._workspace(("muon", gi, shapes), lambda: alloc_workspace(shapes, params[0].device))
        muon_step(params, [p.grad.contiguous() for p in params], moms, lr=group["lr"],
                  mu=group["momentum"], wd=group["wd"], ns_steps=group["ns_steps"],
                  coeffs=group["coeffs"], rms_scale=group["rms_scale"], eps=group["eps"],
                  zero_centering=group["zero_centering"], nesterov=group["nesterov"],
                  ns_first=group["ns_first"], workspace=ws)

    def _step_adamw(self, gi, group):
        params = [p for p in group["params"] if p.grad is not None]
        if not params:
            return
        ms, vs, steps = [], [], []
        for p in params:
            st = self.state[p]
            if "step" not in st:
                st["step"] = 0
                st["exp_avg"] = torch.zeros_like(p)
                st["exp_avg_sq"] = torch.zeros_like(p)
            st["step"] += 1
            ms.append(st["exp_avg"])
            vs.append(st["exp_avg_sq"])
            steps.append(st["step"])
        ws = self._workspace(("adamw", gi, len(params)),
                             lambda: alloc_adamw_workspace(len(params), params[0].device))
        adamw_step(params, [p.grad.contiguous() for p in params], ms, vs, steps, lr=group["adamw_lr"],
                   betas=group["adamw_betas"], eps=group["adamw_eps"], wd=group["wd"], workspace=ws)
