"""The host dispatcher replayed on the CPU (tests/host_replay.cpp): the
library's muon_api.cpp, compiled unchanged with the host compiler against
host stand-ins for the HIP runtime calls and recording kernel launchers, runs
muon_step over the Mamba set, 8 layers of the transformer set, the 2048 ragged
matrices and a mixed list (every kernel class, both orientations, skipped
matrices, per-step coefficients of the hybrid schedule), each list twice and
then with a gradient removed, and over seeded random lists (sides 1 to 4000,
absent gradients, 0 to 12 steps, every accepted variant combination, RMS scale
on or off, through muon_step_ex, a prepared plan or muon_orthogonalize).  The
harness checks the launch sequence, the prefix arrays against the tile counts,
and every descriptor's workspace buffers (inside, aligned, disjoint, sized for
the padded shape) in the table the dispatcher uploaded.  The "finite" case
plants a NaN or infinite value in one norm slot from the momentum stand-in
and checks that MUON_CHECK_FINITE reports it by the caller's matrix index (a
first call, the cached repeat and a plan step), and that nothing is reported
without the variable.  A second build runs the same replay under
AddressSanitizer."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "matrix_aware_optimizer_libmuon_amd", "csrc")


def _build(out, extra=()):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    cmd = [cxx, "-std=c++17", "-O1", "-Wall", *extra, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(ROOT, "tests", "host_replay.cpp"),
           os.path.join(CSRC, "muon_api.cpp"), "-o", out, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    return out


@pytest.fixture(scope="module")
def replay(tmp_path_factory):
    return _build(str(tmp_path_factory.mktemp("replay") / "host_replay"))


def _run(exe, *args):
    r = subprocess.run([exe, *args], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("case", ["mamba", "transformer", "ragged", "mixed", "finite"])
def test_dispatcher_replay(replay, case):
    _run(replay, case)


@pytest.mark.parametrize("seed", range(40))
def test_dispatcher_replay_random_lists(replay, seed):
    _run(replay, "random", str(seed))


def test_dispatcher_replay_under_address_sanitizer(tmp_path):
    exe = _build(str(tmp_path / "host_replay_asan"), ("-fsanitize=address", "-fno-omit-frame-pointer"))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    for args in (["mixed"], ["ragged"], ["finite"], *(["random", str(s)] for s in range(8))):
        r = subprocess.run([exe, *args], capture_output=True, text=True, timeout=300, env=env)
        assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout[-1000:] + r.stderr[-2000:]
