"""The host dispatcher replayed on the CPU (tests/host_replay.cpp): the
library's muon_api.cpp, compiled unchanged with the host compiler against
host stand-ins for the HIP runtime calls and recording kernel launchers, runs
muon_step over the Mamba set, 8 layers of the transformer set, the 2048 ragged
matrices and a mixed list (every kernel class, both orientations, skipped
matrices, per-step coefficients of the hybrid schedule); the harness then
checks the launch sequence, the prefix arrays against the tile counts, and
every descriptor's workspace buffers (inside, aligned, disjoint, sized for the
padded shape) in the table the dispatcher uploaded."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "matrix_aware_optimizer_libmuon_amd", "csrc")


@pytest.fixture(scope="module")
def replay(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("replay") / "host_replay")
    cmd = [cxx, "-std=c++17", "-O1", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(ROOT, "tests", "host_replay.cpp"),
           os.path.join(CSRC, "muon_api.cpp"), "-o", exe, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    return exe


@pytest.mark.parametrize("case", ["mamba", "transformer", "ragged", "mixed"])
def test_dispatcher_replay(replay, case):
    r = subprocess.run([replay, case], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout[-2000:] + r.stderr[-500:]
