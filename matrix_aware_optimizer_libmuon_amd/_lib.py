"""ctypes declarations of the libmuon C ABI (include/muon.h).

Loading is lazy: importing the package works without the library (e.g. to
use the workload generator), but every call into the library fails loudly
when libmuon.so has not been built.  There is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# MUON_LIB selects another build of the same library (e.g. the host
# AddressSanitizer build of build.py --asan); the default is the in-place one.
LIB_PATH = os.environ.get("MUON_LIB") or os.path.join(_HERE, "libmuon.so")

MUON_OK = 0
MUON_EINVAL = -1
MUON_EWORKSPACE = -2
MUON_EHIP = -3
MUON_EALIAS = -4
MUON_ECAPTURE = -5
MUON_ENONFINITE = -6

MUON_F32 = 0
MUON_BF16 = 1

MUON_SCALE_NONE = 0
MUON_SCALE_SQRT_MAX1 = 1

MUON_OPT_ZERO_CENTER = 1
MUON_OPT_NESTEROV = 2
MUON_OPT_NS_FIRST = 4

MUON_PHASES = 8
PHASE_NAMES = ("momentum_norm", "normalize_cast", "gram", "gram2_epilogue", "x_update", "apply",
               "adamw", "ns_fused")

EXPORTED = ("muon_workspace_bytes", "muon_step", "muon_step_ex", "muon_plan_create",
            "muon_plan_step", "muon_plan_destroy", "muon_orthogonalize",
            "muon_workspace_view",
            "muon_adamw_workspace_bytes", "muon_adamw_step",
            "muon_timing_enable", "muon_timing_read", "muon_status_string", "muon_version",
            "muon_step_noalloc", "muon_noalloc_scratch")


class MuonMatrix(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p),
                ("momentum", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("grad_dtype", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class MuonOptions(ctypes.Structure):
    _fields_ = [("flags", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class MuonOrtho(ctypes.Structure):
    _fields_ = [("inp", ctypes.c_void_p), ("out", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("in_dtype", ctypes.c_int32)]


class MuonCoeff(ctypes.Structure):
    _fields_ = [("a", ctypes.c_float), ("b", ctypes.c_float), ("c", ctypes.c_float)]


class MuonAdamWTensor(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p),
                ("exp_avg", ctypes.c_void_p), ("exp_avg_sq", ctypes.c_void_p),
                ("numel", ctypes.c_int64), ("step", ctypes.c_int64),
                ("grad_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class MuonWorkspaceView(ctypes.Structure):
    _fields_ = [("x_off", ctypes.c_size_t * 2), ("a_off", ctypes.c_size_t),
                ("c_off", ctypes.c_size_t), ("c_lo_off", ctypes.c_size_t), ("o_off", ctypes.c_size_t),
                ("nrm2_off", ctypes.c_size_t), ("rows_pad", ctypes.c_int64),
                ("cols_pad", ctypes.c_int64), ("m_pad", ctypes.c_int64),
                ("transposed", ctypes.c_int32), ("tile", ctypes.c_int32)]


_lib = None


class LibMuonError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: libmuon status {status}: {status_string(status)}")


def load() -> ctypes.CDLL:
    """Load libmuon.so (built in place by ``build.py``); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libmuon.so not found at {LIB_PATH}; build it with "
                           "`python -m matrix_aware_optimizer_libmuon_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.muon_workspace_bytes.argtypes = [P(MuonMatrix), ctypes.c_int64]
    lib.muon_workspace_bytes.restype = ctypes.c_size_t
    lib.muon_step.argtypes = [P(MuonMatrix), ctypes.c_int64, ctypes.c_float, ctypes.c_float,
                              ctypes.c_float, ctypes.c_int, P(MuonCoeff), ctypes.c_int, ctypes.c_int,
                              ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.muon_step.restype = ctypes.c_int
    lib.muon_step_ex.argtypes = [P(MuonMatrix), ctypes.c_int64, ctypes.c_float, ctypes.c_float,
                                 ctypes.c_float, ctypes.c_int, P(MuonCoeff), ctypes.c_int,
                                 ctypes.c_int, ctypes.c_float, P(MuonOptions), ctypes.c_void_p,
                                 ctypes.c_size_t, ctypes.c_void_p]
    lib.muon_step_ex.restype = ctypes.c_int
    lib.muon_plan_create.argtypes = [P(MuonMatrix), ctypes.c_int64, ctypes.c_int, P(MuonCoeff),
                                     ctypes.c_int, ctypes.c_int, ctypes.c_float, P(MuonOptions),
                                     ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                     P(ctypes.c_void_p)]
    lib.muon_plan_create.restype = ctypes.c_int
    lib.muon_plan_step.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.muon_plan_step.restype = ctypes.c_int
    lib.muon_plan_destroy.argtypes = [ctypes.c_void_p]
    lib.muon_plan_destroy.restype = None
    lib.muon_orthogonalize.argtypes = [P(MuonOrtho), ctypes.c_int64, ctypes.c_int, P(MuonCoeff),
                                       ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                                       ctypes.c_size_t, ctypes.c_void_p]
    lib.muon_orthogonalize.restype = ctypes.c_int
    lib.muon_workspace_view.argtypes = [P(MuonMatrix), ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                        P(MuonWorkspaceView)]
    lib.muon_workspace_view.restype = ctypes.c_int
    lib.muon_adamw_workspace_bytes.argtypes = [ctypes.c_int64]
    lib.muon_adamw_workspace_bytes.restype = ctypes.c_size_t
    lib.muon_adamw_step.argtypes = [P(MuonAdamWTensor), ctypes.c_int64, ctypes.c_float, ctypes.c_float,
                                    ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_void_p,
                                    ctypes.c_size_t, ctypes.c_void_p]
    lib.muon_adamw_step.restype = ctypes.c_int
    lib.muon_timing_enable.argtypes = [ctypes.c_int]
    lib.muon_timing_enable.restype = ctypes.c_int
    lib.muon_timing_read.argtypes = [P(ctypes.c_double), P(ctypes.c_int64)]
    lib.muon_timing_read.restype = ctypes.c_int
    lib.muon_status_string.argtypes = [ctypes.c_int]
    lib.muon_status_string.restype = ctypes.c_char_p
    lib.muon_step_noalloc.argtypes = [P(MuonMatrix), ctypes.c_int64, ctypes.c_float, ctypes.c_float,
                                      ctypes.c_float, ctypes.c_int, P(MuonCoeff), ctypes.c_int,
                                      ctypes.c_int, ctypes.c_float, ctypes.c_void_p]
    lib.muon_step_noalloc.restype = ctypes.c_int
    lib.muon_noalloc_scratch.argtypes = []
    lib.muon_noalloc_scratch.restype = ctypes.c_void_p
    lib.muon_version.argtypes = []
    lib.muon_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().muon_status_string(int(status)).decode()


def check(status: int, where: str) -> None:
    if status != MUON_OK:
        raise LibMuonError(status, where)
