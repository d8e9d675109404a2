"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/muon.h declares, plans workspaces consistently, and
rejects bad arguments before touching the device."""
import ctypes
import math
import os
import re

import pytest

import matrix_aware_optimizer_libmuon_amd as muon
from matrix_aware_optimizer_libmuon_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from matrix_aware_optimizer_libmuon_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(muon_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert muon.version().startswith("libmuon")


def test_struct_layouts_match_header(lib):
    # sizes the C compiler gives the public structs (LP64)
    assert ctypes.sizeof(muon.MuonMatrix) == 48
    assert ctypes.sizeof(muon.MuonOrtho) == 40
    assert ctypes.sizeof(muon.MuonCoeff) == 12
    assert ctypes.sizeof(muon.MuonWorkspaceView) == 88
    assert ctypes.sizeof(muon.MuonAdamWTensor) == 56


def test_workspace_plan(lib):
    shapes = [(256, 768), (1536, 80), (48, 1536), (1, 1), (300, 300)]
    total = muon.workspace_bytes(shapes)
    views = [muon.workspace_view(shapes, i, 5) for i in range(len(shapes))]
    end = 0
    for (r, c), v in zip(shapes, views):
        t = v["tile"]
        assert v["rows_pad"] == math.ceil(r / t) * t and v["cols_pad"] == math.ceil(c / t) * t
        assert v["transposed"] == (r > c)
        assert v["m_pad"] == (v["cols_pad"] if r > c else v["rows_pad"])
        xb = v["rows_pad"] * v["cols_pad"] * 2
        ab = v["m_pad"] ** 2 * 2
        assert v["x_off"][0] % 256 == 0 and v["x_off"][0] >= end
        assert v["x_off"][1] >= v["x_off"][0] + xb
        assert v["a_off"] >= v["x_off"][1] + xb and v["c_off"] >= v["a_off"] + ab
        assert v["o_off"] == v["x_off"][1]          # 5 iterations end in the odd buffer
        end = v["c_off"] + ab
        if min(r, c) <= 128:                         # short side <= 128: low part of C kept
            assert v["c_lo_off"] >= end
            end = v["c_lo_off"] + ab
        else:
            assert v["c_lo_off"] == 0
    assert end <= total
    assert muon.workspace_view(shapes, 0, 4)["o_off"] == views[0]["x_off"][0]
    nrm = [v["nrm2_off"] for v in views]
    assert all(b - a == 8 for a, b in zip(nrm, nrm[1:])) and nrm[-1] + 8 <= views[0]["x_off"][0]


def test_workspace_rejects_bad_shapes(lib):
    with pytest.raises(ValueError):
        muon.workspace_bytes([(0, 5)])
    with pytest.raises(ValueError):
        muon.workspace_bytes([(5, (1 << 20) + 1)])
    assert muon.workspace_bytes([]) == 0


def _mats(specs):
    arr = (muon.MuonMatrix * len(specs))()
    for i, s in enumerate(specs):
        for k, v in s.items():
            setattr(arr[i], k, v)
    return arr


def _call(lib, arr, n, *, ns=5, coeffs=((3.4445, -4.775, 2.0315),), eps=1e-7, lr=0.02, mu=0.95,
          wd=0.0, mode=0, ws=1 << 40, ws_bytes=1 << 60):
    carr = (muon.MuonCoeff * max(1, len(coeffs)))(*[muon.MuonCoeff(*c) for c in coeffs])
    return lib.muon_step(arr, n, lr, mu, wd, ns, carr if coeffs else None, len(coeffs), mode, eps,
                         ctypes.c_void_p(ws), ws_bytes, None)


GOOD = dict(param=0x10000000, grad=0x20000000, momentum=0x30000000, rows=64, cols=64,
            grad_dtype=muon.MUON_BF16)


def test_argument_errors_are_caught_on_the_host(lib):
    ok = _mats([GOOD])
    assert _call(lib, ok, 1, ns=-1) == muon.MUON_EINVAL
    assert _call(lib, ok, 1, ns=65) == muon.MUON_EINVAL
    assert _call(lib, ok, 1, coeffs=((1, 2, 3), (1, 2, 3))) == muon.MUON_EINVAL
    assert _call(lib, ok, 1, eps=-1.0) == muon.MUON_EINVAL
    assert _call(lib, ok, 1, lr=float("nan")) == muon.MUON_EINVAL
    assert _call(lib, ok, 1, mode=7) == muon.MUON_EINVAL
    assert _call(lib, ok, 1, coeffs=((float("inf"), 0, 0),)) == muon.MUON_EINVAL
    assert _call(lib, ok, -1) == muon.MUON_EINVAL
    assert _call(lib, _mats([dict(GOOD, rows=0)]), 1) == muon.MUON_EINVAL
    assert _call(lib, _mats([dict(GOOD, param=0)]), 1) == muon.MUON_EINVAL
    assert _call(lib, _mats([dict(GOOD, momentum=0)]), 1) == muon.MUON_EINVAL
    assert _call(lib, _mats([dict(GOOD, grad_dtype=5)]), 1) == muon.MUON_EINVAL
    assert _call(lib, _mats([dict(GOOD, param=0x10000002)]), 1) == muon.MUON_EINVAL


def test_aliasing_is_rejected(lib):
    # momentum overlapping the param, and two matrices sharing a param
    assert _call(lib, _mats([dict(GOOD, momentum=GOOD["param"] + 64)]), 1) == muon.MUON_EALIAS
    two = _mats([GOOD, dict(GOOD, grad=0x40000000, momentum=0x50000000)])
    assert _call(lib, two, 2) == muon.MUON_EALIAS


def test_workspace_errors(lib):
    ok = _mats([GOOD])
    need = lib.muon_workspace_bytes(ok, 1)
    assert need > 0
    assert _call(lib, ok, 1, ws=1 << 40, ws_bytes=need - 1) == muon.MUON_EWORKSPACE
    assert _call(lib, ok, 1, ws=(1 << 40) + 16, ws_bytes=need) == muon.MUON_EWORKSPACE
    assert _call(lib, ok, 1, ws=0, ws_bytes=need) == muon.MUON_EWORKSPACE


def test_nothing_to_do_returns_ok_without_device(lib):
    # all gradients absent: validated, then nothing is launched
    skipped = _mats([dict(GOOD, grad=0)])
    assert _call(lib, skipped, 1) == muon.MUON_OK
    assert _call(lib, skipped, 0) == muon.MUON_OK


def test_orthogonalize_argument_errors(lib):
    arr = (muon.MuonOrtho * 1)()
    arr[0].inp, arr[0].out, arr[0].rows, arr[0].cols, arr[0].in_dtype = 0x1000, 0x100000, 8, 8, 0
    c = (muon.MuonCoeff * 1)(muon.MuonCoeff(3.4445, -4.775, 2.0315))
    assert lib.muon_orthogonalize(arr, 1, 5, c, 2, 1e-7, ctypes.c_void_p(1 << 40), 1 << 40, None) == muon.MUON_EINVAL
    arr[0].out = 0x1000 + 64
    assert lib.muon_orthogonalize(arr, 1, 5, c, 1, 1e-7, ctypes.c_void_p(1 << 40), 1 << 40, None) == muon.MUON_EALIAS
    arr[0].out = 0
    assert lib.muon_orthogonalize(arr, 1, 5, c, 1, 1e-7, ctypes.c_void_p(1 << 40), 1 << 40, None) == muon.MUON_EINVAL


def test_status_strings(lib):
    for st in (muon.MUON_OK, muon.MUON_EINVAL, muon.MUON_EWORKSPACE, muon.MUON_EALIAS, muon.MUON_EHIP,
               muon.MUON_ECAPTURE, muon.MUON_ENONFINITE, -99):
        assert isinstance(muon.status_string(st), str) and muon.status_string(st)
    assert "captur" in muon.status_string(muon.MUON_ECAPTURE)
    assert "non-finite" in muon.status_string(muon.MUON_ENONFINITE)
    # the binding's status values are the header's
    header = open(os.path.join(ROOT, "include", "muon.h")).read()
    for name in ("MUON_OK", "MUON_EINVAL", "MUON_EWORKSPACE", "MUON_EHIP", "MUON_EALIAS",
                 "MUON_ECAPTURE", "MUON_ENONFINITE"):
        m = re.search(r"#define\s+" + name + r"\s+(-?\d+)", header)
        assert m and int(m.group(1)) == getattr(muon, name), name
    with pytest.raises(muon.LibMuonError):
        _lib.check(muon.MUON_EINVAL, "x")


def test_python_binding_validates_before_calling(lib):
    torch = pytest.importorskip("torch")
    p = torch.zeros(4, 4)
    with pytest.raises(ValueError):
        muon.muon_step([p], [p], [p])                 # CPU tensors are refused
    with pytest.raises(ValueError):
        muon.muon_step([p], [p], [])


def _adam(specs):
    arr = (muon.MuonAdamWTensor * max(1, len(specs)))()
    for i, s in enumerate(specs):
        for k, v in s.items():
            setattr(arr[i], k, v)
    return arr


AGOOD = dict(param=0x10000000, grad=0x20000000, exp_avg=0x30000000, exp_avg_sq=0x40000000,
             numel=1000, step=1, grad_dtype=muon.MUON_F32)


def _acall(lib, arr, n, *, lr=1e-3, b1=0.9, b2=0.95, eps=1e-8, wd=0.01, ws=1 << 40, ws_bytes=1 << 30):
    return lib.muon_adamw_step(arr, n, lr, b1, b2, eps, wd, ctypes.c_void_p(ws), ws_bytes, None)


def test_adamw_argument_errors_are_caught_on_the_host(lib):
    ok = _adam([AGOOD])
    assert lib.muon_adamw_workspace_bytes(0) == 0 and lib.muon_adamw_workspace_bytes(3) > 0
    assert _acall(lib, ok, 1, b1=1.0) == muon.MUON_EINVAL
    assert _acall(lib, ok, 1, b2=-0.1) == muon.MUON_EINVAL
    assert _acall(lib, ok, 1, eps=-1.0) == muon.MUON_EINVAL
    assert _acall(lib, ok, 1, lr=float("inf")) == muon.MUON_EINVAL
    assert _acall(lib, ok, -1) == muon.MUON_EINVAL
    assert _acall(lib, _adam([dict(AGOOD, numel=0)]), 1) == muon.MUON_EINVAL
    assert _acall(lib, _adam([dict(AGOOD, step=0)]), 1) == muon.MUON_EINVAL
    assert _acall(lib, _adam([dict(AGOOD, reserved=1)]), 1) == muon.MUON_EINVAL
    assert _acall(lib, _adam([dict(AGOOD, exp_avg=0)]), 1) == muon.MUON_EINVAL
    assert _acall(lib, _adam([dict(AGOOD, grad_dtype=3)]), 1) == muon.MUON_EINVAL
    assert _acall(lib, _adam([dict(AGOOD, param=0x10000002)]), 1) == muon.MUON_EINVAL
    # second moment overlapping the param; two tensors sharing a first moment
    assert _acall(lib, _adam([dict(AGOOD, exp_avg_sq=AGOOD["param"] + 400)]), 1) == muon.MUON_EALIAS
    two = _adam([AGOOD, dict(AGOOD, param=0x50000000, grad=0x60000000, exp_avg_sq=0x70000000)])
    assert _acall(lib, two, 2) == muon.MUON_EALIAS
    need = lib.muon_adamw_workspace_bytes(1)
    assert _acall(lib, ok, 1, ws_bytes=need - 1) == muon.MUON_EWORKSPACE
    assert _acall(lib, ok, 1, ws=(1 << 40) + 8, ws_bytes=need) == muon.MUON_EWORKSPACE
    # no gradients: validated, nothing launched
    assert _acall(lib, _adam([dict(AGOOD, grad=0, step=0)]), 1) == muon.MUON_OK
    assert _acall(lib, ok, 0) == muon.MUON_OK


def test_step_variant_options_are_validated(lib):
    ok = _mats([GOOD])
    c = (muon.MuonCoeff * 1)(muon.MuonCoeff(3.4445, -4.775, 2.0315))

    def call(flags, reserved=0, ws_bytes=1 << 60):
        opts = muon.MuonOptions(flags, reserved)
        return lib.muon_step_ex(ok, 1, 0.02, 0.95, 0.0, 5, c, 1, 0, 1e-7, ctypes.byref(opts),
                                ctypes.c_void_p(1 << 40), ws_bytes, None)

    assert call(8) == muon.MUON_EINVAL                                   # unknown flag
    assert call(muon.MUON_OPT_ZERO_CENTER, reserved=1) == muon.MUON_EINVAL
    assert call(muon.MUON_OPT_NESTEROV | muon.MUON_OPT_NS_FIRST) == muon.MUON_EINVAL
    # valid options still meet the workspace check before any launch
    for f in (muon.MUON_OPT_ZERO_CENTER, muon.MUON_OPT_NESTEROV, muon.MUON_OPT_NS_FIRST,
              muon.MUON_OPT_ZERO_CENTER | muon.MUON_OPT_NS_FIRST):
        assert call(f, ws_bytes=16) == muon.MUON_EWORKSPACE
    # NULL options: the plain step's validation
    assert lib.muon_step_ex(ok, 1, 0.02, 0.95, 0.0, -1, c, 1, 0, 1e-7, None,
                            ctypes.c_void_p(1 << 40), 1 << 60, None) == muon.MUON_EINVAL


def test_workspace_reserves_column_sums(lib):
    # the column-sum region sits between the table and the first X buffer
    shapes = [(300, 2100), (7, 9)]
    v0 = muon.workspace_view(shapes, 0, 5)
    assert v0["x_off"][0] >= v0["nrm2_off"] + 16 + 8 * (2100 + 9)


def test_marshalling_module_matches_the_header(lib):
    m = muon._marshaller()
    assert m.MATRIX_BYTES == ctypes.sizeof(muon.MuonMatrix)
    assert m.ORTHO_BYTES == ctypes.sizeof(muon.MuonOrtho)
    assert m.ADAMW_BYTES == ctypes.sizeof(muon.MuonAdamWTensor)


def test_marshalling_rejects_bad_tensors(lib):
    torch = pytest.importorskip("torch")
    m = muon._marshaller()
    arr = (muon.MuonMatrix * 2)()
    p = torch.zeros(4, 4)
    with pytest.raises(ValueError, match="same length"):
        m.fill_matrices([p], [p, p], [p], [], ctypes.addressof(arr))
    with pytest.raises(ValueError, match="scales"):
        m.fill_matrices([p], [p], [p], [1.0, 2.0], ctypes.addressof(arr))
    with pytest.raises(ValueError, match=r"params\[0\] must be 2-D"):
        m.fill_matrices([torch.zeros(4)], [None], [torch.zeros(4)], [], ctypes.addressof(arr))
    with pytest.raises(ValueError, match=r"params\[0\] must be contiguous"):
        m.fill_matrices([p.t()[:, :2]], [None], [p], [], ctypes.addressof(arr))
    with pytest.raises(ValueError, match="GPU"):
        m.fill_matrices([p], [p], [p], [], ctypes.addressof(arr))
    with pytest.raises(ValueError, match="same length"):
        m.fill_adamw([p], [p], [p], [p], [1, 2], ctypes.addressof(arr))
    with pytest.raises(ValueError, match="same length"):
        m.fill_ortho([p], [], ctypes.addressof(arr))
    assert m.fill_matrices([], [], [], [], ctypes.addressof(arr)) is None


def test_kernel_class_by_shape(lib):
    # fused: short side <= 128 and, padded to 32 with LDS rows of 128
    # elements, m n + 2 m m bf16 within 160 KB; 256 from a short side of 1024
    def tile(r, c):
        return muon.workspace_view([(r, c)], 0, 5)["tile"]

    def lds(r, c):
        m, n = -(-min(r, c) // 32) * 32, -(-max(r, c) // 32) * 32
        return 2 * (m * (-(-n // 128) * 128) + 2 * m * (-(-m // 128) * 128))

    for r, c in [(1, 1), (1, 40), (40, 1), (17, 15), (64, 1024), (1024, 64), (100, 300),
                 (300, 100), (128, 256), (48, 1000), (32, 2304)]:
        assert lds(r, c) <= 160 * 1024 and tile(r, c) == 32, (r, c)
    for r, c in [(64, 1056), (129, 257), (128, 512), (48, 1536), (1536, 80), (256, 768)]:
        assert tile(r, c) == 128, (r, c)
    assert tile(1024, 1024) == 256 and tile(4096, 14336) == 256
    v = muon.workspace_view([(100, 300)], 0, 5)
    assert (v["rows_pad"], v["cols_pad"], v["m_pad"]) == (128, 320, 128)


def test_plan_arguments_are_validated_on_the_host(lib):
    ok = _mats([GOOD])
    c = (muon.MuonCoeff * 1)(muon.MuonCoeff(3.4445, -4.775, 2.0315))
    out = ctypes.c_void_p()

    def create(arr, n, *, ns=5, ws_bytes=1 << 60, out_ptr=True, opts=None):
        return lib.muon_plan_create(arr, n, ns, c, 1, 0, 1e-7, opts, ctypes.c_void_p(1 << 40), ws_bytes,
                                    None, ctypes.byref(out) if out_ptr else None)

    assert create(ok, 1, out_ptr=False) == muon.MUON_EINVAL
    assert create(ok, 1, ns=-1) == muon.MUON_EINVAL
    assert create(ok, 1, ws_bytes=16) == muon.MUON_EWORKSPACE
    assert create(_mats([dict(GOOD, momentum=GOOD["param"] + 64)]), 1) == muon.MUON_EALIAS
    bad = muon.MuonOptions(muon.MUON_OPT_NESTEROV | muon.MUON_OPT_NS_FIRST, 0)
    assert create(ok, 1, opts=ctypes.byref(bad)) == muon.MUON_EINVAL
    assert out.value is None                         # nothing was created
    assert lib.muon_plan_step(None, ctypes.c_void_p(1 << 40), None) == muon.MUON_EINVAL
    lib.muon_plan_destroy(None)                      # a no-op


def test_workspace_buffers_are_disjoint_and_inside(lib):
    """For seeded random lists mixing every kernel class (fused 32..128, tile
    128, tile 256; wide, tall, square, ragged), every matrix's buffers --
    two iterates, A, C and (short side <= 128) C_lo -- lie inside the
    workspace, after the table, 256-byte aligned, and overlap nothing else:
    the kernels of different matrices (and the fused class, which runs on its
    own stream beside the tiled classes) never write the same bytes."""
    import random
    rng = random.Random(1234)
    sides = [1, 7, 31, 33, 64, 100, 128, 129, 200, 256, 511, 768, 1024, 1100, 1536, 2304]
    for trial in range(12):
        shapes = [(rng.choice(sides), rng.choice(sides)) for _ in range(rng.randint(1, 24))]
        total = muon.workspace_bytes(shapes)
        spans = []
        first = None
        for i, (r, c) in enumerate(shapes):
            v = muon.workspace_view(shapes, i, 5)
            xb = v["rows_pad"] * v["cols_pad"] * 2
            ab = v["m_pad"] ** 2 * 2
            assert v["rows_pad"] >= r and v["cols_pad"] >= c
            assert v["m_pad"] == min(v["rows_pad"], v["cols_pad"]) or v["tile"] != 32
            bufs = [(v["x_off"][0], xb), (v["x_off"][1], xb), (v["a_off"], ab), (v["c_off"], ab)]
            if v["c_lo_off"]:
                bufs.append((v["c_lo_off"], ab))
            for off, size in bufs:
                assert off % 256 == 0 and 0 < off and off + size <= total, (trial, i, off, size)
                spans.append((off, off + size, i))
            first = min(first, min(o for o, _ in bufs)) if first is not None else min(o for o, _ in bufs)
            assert v["nrm2_off"] + 8 <= first
        spans.sort()
        for (a0, a1, ia), (b0, b1, ib) in zip(spans, spans[1:]):
            assert a1 <= b0, f"trial {trial}: buffers of matrices {ia} and {ib} overlap"
