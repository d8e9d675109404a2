"""libmuon for MI355X: the Muon optimizer step as hand-written gfx950 kernels
behind a C ABI (include/muon.h).  This module only marshals arguments: every
step of the computation runs in libmuon.so.  PyTorch supplies device memory
and the stream.

    import torch
    import matrix_aware_optimizer_libmuon_amd as muon
    ws = muon.alloc_workspace([p.shape for p in params], device="cuda")
    muon.muon_step(params, grads, moms, lr=0.02, mu=0.95, wd=0.01, workspace=ws)
"""
from __future__ import annotations

import ctypes
from typing import Iterable, Sequence

from . import _lib
from ._lib import (MUON_BF16, MUON_EALIAS, MUON_ECAPTURE, MUON_EHIP, MUON_EINVAL,  # noqa: F401
                   MUON_ENONFINITE, MUON_EWORKSPACE,
                   MUON_F32, MUON_OK, MUON_OPT_NESTEROV, MUON_OPT_NS_FIRST, MUON_OPT_ZERO_CENTER,
                   MuonOptions, MUON_SCALE_NONE, MUON_SCALE_SQRT_MAX1, PHASE_NAMES,
                   LibMuonError, MuonAdamWTensor, MuonCoeff, MuonMatrix, MuonOrtho,
                   MuonWorkspaceView, status_string)

# Quintic Newton-Schulz coefficients (a, b, c) of the newtonschulz5 routine in
# "Muon optimizer: matrix-aware LLM" (airosetta.com, implementation section).
QUINTIC = (3.4445, -4.7750, 2.0315)
# "AdamW vs Muon" (adg.csdn.net), section "3. DeepSeek-V4 hybrid schedule":
# 8 quintic steps then 2 steps of (2, -1.5, 0.5).
HYBRID = [QUINTIC] * 8 + [(2.0, -1.5, 0.5)] * 2


def version() -> str:
    return _lib.load().muon_version().decode()


def _torch():
    import torch
    return torch


_MARSHAL = None


def _marshaller():
    """The C++ marshalling module (fills descriptor arrays from tensor lists)."""
    global _MARSHAL
    if _MARSHAL is None:
        _torch()  # its shared libraries must be loaded first
        try:
            from . import _marshal as m
        except ImportError as e:
            raise RuntimeError("the binding's marshalling module is not built; build it with "
                               "`python -m matrix_aware_optimizer_libmuon_amd.build`") from e
        _MARSHAL = m
    return _MARSHAL


def _coeff_array(coeffs, ns_steps: int):
    if coeffs is None:
        coeffs = QUINTIC
    if len(coeffs) == 3 and not isinstance(coeffs[0], (tuple, list)):
        coeffs = [tuple(coeffs)]
    coeffs = [tuple(float(v) for v in c) for c in coeffs]
    arr = (MuonCoeff * max(1, len(coeffs)))(*[MuonCoeff(*c) for c in coeffs])
    return arr, len(coeffs)


def _shapes_array(shapes: Sequence) -> ctypes.Array:
    arr = (MuonMatrix * max(1, len(shapes)))()
    for i, (r, c) in enumerate(shapes):
        arr[i].rows = int(r)
        arr[i].cols = int(c)
    return arr


def workspace_bytes(shapes: Sequence) -> int:
    """Workspace bytes for a list of (rows, cols)."""
    shapes = [tuple(int(v) for v in s) for s in shapes]
    if not shapes:
        return 0
    n = _lib.load().muon_workspace_bytes(_shapes_array(shapes), len(shapes))
    if n == 0:
        raise ValueError("invalid shape list")
    return int(n)


def alloc_workspace(shapes: Sequence, device="cuda"):
    """A uint8 device tensor big enough for ``shapes`` (256-byte aligned)."""
    torch = _torch()
    n = workspace_bytes(shapes)
    ws = torch.empty(max(n, 256) + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + max(n, 256)]


def workspace_view(shapes: Sequence, index: int, ns_steps: int) -> dict:
    """Byte offsets of matrix ``index``'s intermediates in the workspace."""
    shapes = [tuple(int(v) for v in s) for s in shapes]
    v = MuonWorkspaceView()
    _lib.check(_lib.load().muon_workspace_view(_shapes_array(shapes), len(shapes), int(index),
                                               int(ns_steps), ctypes.byref(v)),
               "muon_workspace_view")
    return {"x_off": (v.x_off[0], v.x_off[1]), "a_off": v.a_off, "c_off": v.c_off,
            "c_lo_off": v.c_lo_off,
            "o_off": v.o_off, "nrm2_off": v.nrm2_off, "rows_pad": v.rows_pad,
            "cols_pad": v.cols_pad, "m_pad": v.m_pad, "transposed": bool(v.transposed),
            "tile": v.tile}


def _on(device):
    """The tensors' device as the current one for the duration of a library
    call (the library works on the calling thread's current device)."""
    return _torch().cuda.device(device)


def _stream_handle(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(int(stream.cuda_stream))


def muon_step(params: Sequence, grads: Sequence, moms: Sequence, *, lr: float = 0.02,
              mu: float = 0.95, wd: float = 0.0, ns_steps: int = 5, coeffs=QUINTIC,
              rms_scale: str | None = None, eps: float = 1e-7, scales: Sequence | None = None,
              zero_centering: bool = False, nesterov: bool = False, ns_first: bool = False,
              workspace=None, stream=None):
    """One Muon step over lists of 2-D fp32 params, grads (fp32 or bf16, or
    None to skip) and fp32 momentum buffers, all on one GPU.  Updates params
    and momenta in place on ``stream`` (default: the current stream) and
    returns the workspace tensor used.  ``zero_centering``, ``nesterov`` and
    ``ns_first`` select the step variants of ``muon_step_ex``."""
    torch = _torch()
    n = len(params)
    if rms_scale not in (None, "none", "sqrt_max1"):
        raise ValueError(f"unknown rms_scale {rms_scale!r}")
    mode = MUON_SCALE_SQRT_MAX1 if rms_scale == "sqrt_max1" else MUON_SCALE_NONE
    arr = (MuonMatrix * max(1, n))()
    sc = [] if scales is None else [0.0 if s is None else float(s) for s in scales]
    _marshaller().fill_matrices(params, grads, moms, sc, ctypes.addressof(arr))
    device = params[0].device if n else torch.device("cuda")
    if workspace is None:
        workspace = alloc_workspace([tuple(p.shape) for p in params], device)
    carr, nc = _coeff_array(coeffs, ns_steps)
    flags = ((MUON_OPT_ZERO_CENTER if zero_centering else 0) | (MUON_OPT_NESTEROV if nesterov else 0)
             | (MUON_OPT_NS_FIRST if ns_first else 0))
    lib = _lib.load()
    ws_args = (ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
               _stream_handle(stream, device))
    with _on(device):
        if flags:
            opts = MuonOptions(flags, 0)
            st = lib.muon_step_ex(arr, n, float(lr), float(mu), float(wd), int(ns_steps), carr, nc,
                                  mode, float(eps), ctypes.byref(opts), *ws_args)
        else:
            st = lib.muon_step(arr, n, float(lr), float(mu), float(wd), int(ns_steps), carr, nc,
                               mode, float(eps), *ws_args)
    _lib.check(st, "muon_step")
    return workspace


# Bytes of the fixed per-device scratch of muon_step_noalloc (include/muon.h).
NOALLOC_SCRATCH_BYTES = 64 << 20


def muon_step_noalloc(params: Sequence, grads: Sequence, moms: Sequence, *, lr: float = 0.02,
                      mu: float = 0.95, wd: float = 0.0, ns_steps: int = 5, coeffs=QUINTIC,
                      rms_scale: str | None = None, eps: float = 1e-7,
                      scales: Sequence | None = None, stream=None) -> None:
    """muon_step without a workspace and without any allocation
    (``muon_step_noalloc``): the intermediates live in the library's fixed
    per-device scratch of NOALLOC_SCRATCH_BYTES, shared by every such call on
    the device (calls that overlap on one device race)."""
    torch = _torch()
    n = len(params)
    if rms_scale not in (None, "none", "sqrt_max1"):
        raise ValueError(f"unknown rms_scale {rms_scale!r}")
    mode = MUON_SCALE_SQRT_MAX1 if rms_scale == "sqrt_max1" else MUON_SCALE_NONE
    arr = (MuonMatrix * max(1, n))()
    sc = [] if scales is None else [0.0 if s is None else float(s) for s in scales]
    _marshaller().fill_matrices(params, grads, moms, sc, ctypes.addressof(arr))
    device = params[0].device if n else torch.device("cuda")
    carr, nc = _coeff_array(coeffs, ns_steps)
    with _on(device):
        st = _lib.load().muon_step_noalloc(arr, n, float(lr), float(mu), float(wd), int(ns_steps),
                                           carr, nc, mode, float(eps), _stream_handle(stream, device))
    _lib.check(st, "muon_step_noalloc")


class Plan:
    """A Muon step prepared once over fixed tensors (``muon_plan_create``):
    ``step()`` then only launches kernels, so it can be captured into a CUDA
    (HIP) graph and replayed.  Write new gradients into the same grad tensors
    between steps; ``lr``, ``mu`` and ``wd`` live in the device tensor
    ``hyper`` ({lr, mu, wd}, float32), read by the kernels when they run, so
    ``set_hyper`` follows a schedule across replays.  The tensors and the
    workspace are kept alive by the plan."""

    def __init__(self, params: Sequence, grads: Sequence, moms: Sequence, *, lr: float = 0.02,
                 mu: float = 0.95, wd: float = 0.0, ns_steps: int = 5, coeffs=QUINTIC,
                 rms_scale: str | None = None, eps: float = 1e-7, scales: Sequence | None = None,
                 zero_centering: bool = False, nesterov: bool = False, ns_first: bool = False,
                 workspace=None, stream=None):
        torch = _torch()
        n = len(params)
        if rms_scale not in (None, "none", "sqrt_max1"):
            raise ValueError(f"unknown rms_scale {rms_scale!r}")
        mode = MUON_SCALE_SQRT_MAX1 if rms_scale == "sqrt_max1" else MUON_SCALE_NONE
        arr = (MuonMatrix * max(1, n))()
        sc = [] if scales is None else [0.0 if s is None else float(s) for s in scales]
        _marshaller().fill_matrices(params, grads, moms, sc, ctypes.addressof(arr))
        self.device = params[0].device if n else torch.device("cuda")
        self.tensors = (list(params), list(grads), list(moms))
        if workspace is None:
            workspace = alloc_workspace([tuple(p.shape) for p in params], self.device)
        self.workspace = workspace
        self.hyper = torch.tensor([lr, mu, wd], dtype=torch.float32, device=self.device)
        flags = ((MUON_OPT_ZERO_CENTER if zero_centering else 0)
                 | (MUON_OPT_NESTEROV if nesterov else 0) | (MUON_OPT_NS_FIRST if ns_first else 0))
        opts = MuonOptions(flags, 0)
        carr, nc = _coeff_array(coeffs, ns_steps)
        self._lib = _lib.load()
        handle = ctypes.c_void_p()
        with _on(self.device):
            st = self._lib.muon_plan_create(arr, n, int(ns_steps), carr, nc, mode, float(eps),
                                            ctypes.byref(opts), ctypes.c_void_p(workspace.data_ptr()),
                                            workspace.numel() * workspace.element_size(),
                                            _stream_handle(stream, self.device), ctypes.byref(handle))
        _lib.check(st, "muon_plan_create")
        self._handle = handle

    def set_hyper(self, lr: float | None = None, mu: float | None = None,
                  wd: float | None = None) -> None:
        """Stream-ordered update of {lr, mu, wd} on the device."""
        for k, v in enumerate((lr, mu, wd)):
            if v is not None:
                self.hyper[k] = float(v)

    def step(self, stream=None) -> None:
        if not self._handle:
            raise RuntimeError("plan is closed")
        with _on(self.device):
            st = self._lib.muon_plan_step(self._handle, ctypes.c_void_p(self.hyper.data_ptr()),
                                          _stream_handle(stream, self.device))
        _lib.check(st, "muon_plan_step")

    def close(self) -> None:
        if getattr(self, "_handle", None):
            self._lib.muon_plan_destroy(self._handle)
            self._handle = None

    def __del__(self):
        self.close()


def orthogonalize(inputs: Sequence, outputs: Sequence | None = None, *, ns_steps: int = 5,
                  coeffs=QUINTIC, eps: float = 1e-7, workspace=None, stream=None):
    """out_i = NS(in_i) in bf16 for a list of 2-D fp32/bf16 GPU tensors.
    Returns the list of bf16 outputs (allocated when not given)."""
    torch = _torch()
    n = len(inputs)
    device = inputs[0].device if n else torch.device("cuda")
    if outputs is None:
        outputs = [torch.empty(t.shape, dtype=torch.bfloat16, device=t.device) for t in inputs]
    arr = (MuonOrtho * max(1, n))()
    _marshaller().fill_ortho(inputs, outputs, ctypes.addressof(arr))
    if workspace is None:
        workspace = alloc_workspace([tuple(t.shape) for t in inputs], device)
    carr, nc = _coeff_array(coeffs, ns_steps)
    with _on(device):
        st = _lib.load().muon_orthogonalize(arr, n, int(ns_steps), carr, nc, float(eps),
                                            ctypes.c_void_p(workspace.data_ptr()),
                                            workspace.numel() * workspace.element_size(),
                                            _stream_handle(stream, device))
    _lib.check(st, "muon_orthogonalize")
    return outputs


# AdamW defaults of the optimizer constructor in "Muon meets Mamba" (wmrh.cn),
# section 4.1: adamw_lr, adamw_betas, adamw_eps, and the shared weight decay.
ADAMW_DEFAULTS = {"lr": 1e-3, "betas": (0.9, 0.95), "eps": 1e-8, "wd": 0.01}


def adamw_workspace_bytes(n_tensors: int) -> int:
    return int(_lib.load().muon_adamw_workspace_bytes(int(n_tensors)))


def alloc_adamw_workspace(n_tensors: int, device="cuda"):
    torch = _torch()
    n = max(adamw_workspace_bytes(n_tensors), 256)
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + n]


def adamw_step(params: Sequence, grads: Sequence, exp_avgs: Sequence, exp_avg_sqs: Sequence,
               steps: Sequence, *, lr: float = 1e-3, betas=(0.9, 0.95), eps: float = 1e-8,
               wd: float = 0.01, workspace=None, stream=None):
    """One AdamW update of fp32 GPU tensors of any shape (grads fp32 or bf16,
    or None to skip), in place, one grouped launch.  ``steps[i]`` is tensor
    i's step count for this update (>= 1); the caller keeps and increments
    it.  Returns the workspace used."""
    torch = _torch()
    n = len(params)
    arr = (MuonAdamWTensor * max(1, n))()
    _marshaller().fill_adamw(params, grads, exp_avgs, exp_avg_sqs, [int(t) for t in steps],
                          ctypes.addressof(arr))
    device = params[0].device if n else torch.device("cuda")
    if workspace is None:
        workspace = alloc_adamw_workspace(n, device)
    with _on(device):
        st = _lib.load().muon_adamw_step(arr, n, float(lr), float(betas[0]), float(betas[1]),
                                         float(eps), float(wd), ctypes.c_void_p(workspace.data_ptr()),
                                         workspace.numel() * workspace.element_size(),
                                         _stream_handle(stream, device))
    _lib.check(st, "muon_adamw_step")
    return workspace


def timing_enable(on: bool = True) -> None:
    _lib.check(_lib.load().muon_timing_enable(1 if on else 0), "muon_timing_enable")


def timing_read() -> dict:
    """Per-phase summed milliseconds and launch counts since the last read
    (waits for the recorded events)."""
    ms = (ctypes.c_double * _lib.MUON_PHASES)()
    cnt = (ctypes.c_int64 * _lib.MUON_PHASES)()
    _lib.check(_lib.load().muon_timing_read(ms, cnt), "muon_timing_read")
    return {name: {"ms": ms[k], "launches": cnt[k]} for k, name in enumerate(PHASE_NAMES)}
