"""The host side of the library under AddressSanitizer (CPU only).

Builds libmuon with its host dispatcher instrumented (build.py --asan; the
device code is unchanged and never runs here), then runs the host test files
against that build in a child process with the sanitizer runtime preloaded.
Any heap overflow, use after free or double free in argument checking,
workspace planning, descriptor tables or the staging ring fails the child."""
import os
import subprocess
import sys

import pytest

from matrix_aware_optimizer_libmuon_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_TESTS = ["tests/test_host.py", "tests/test_optim_host.py", "tests/test_profiling.py"]


@pytest.mark.timeout(600)
def test_host_code_is_clean_under_address_sanitizer(tmp_path):
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in the ROCm toolchain")
    lib = build.build_asan(str(tmp_path / "asan"))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms          # the host code really is instrumented
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["MUON_LIB"] = lib
    env.pop("PYTEST_XDIST_WORKER", None)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *HOST_TESTS], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=540)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr, tail
    assert " passed" in r.stdout, tail
    # the child ran the instrumented build, not the in-place one
    probe = subprocess.run([sys.executable, "-c",
                            "from matrix_aware_optimizer_libmuon_amd import _lib; print(_lib.LIB_PATH)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert probe.stdout.strip() == lib, probe.stdout + probe.stderr
