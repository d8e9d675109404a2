"""Host logic of bench.py that needs no GPU: the one-GPU refusal, the
algorithmic work per phase it divides by, and the CPU-baseline leg (the
fp64 oracle on a bounded sample)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from matrix_aware_optimizer_libmuon_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


class _ClassOf:
    """Stand-in for the library's workspace_view: the kernel class by shape
    (fused below a short side of 128, else a tiled class)."""

    @staticmethod
    def workspace_view(shapes, index, ns_steps):
        r, c = shapes[index]
        return {"tile": bench.FUSED_TILE if min(r, c) <= 128 else 256}


def test_phase_work_closed_forms():
    w = W.WORKLOADS[3]                        # transformer set: every matrix tiled
    work = bench.phase_work(w, _ClassOf)
    e = sum(r * c for r, c in w.shapes)
    assert work["momentum_norm"] == ("hbm", e * (2 + 8))     # bf16 G, fp32 M read + write
    assert work["normalize_cast"] == ("hbm", e * 6)
    assert work["apply"] == ("hbm", e * 10)
    gram = sum(2 * min(s) ** 2 * max(s) for s in w.shapes)
    assert work["gram"] == ("mfma", gram) and work["x_update"] == ("mfma", gram)
    assert work["gram2_epilogue"] == ("mfma", sum(2 * min(s) ** 3 for s in w.shapes))
    assert work["ns_fused"] == ("mfma", 0)
    # one launch per phase and iteration: the tiled phases times ns_steps add up
    # to the workload's nominal Newton-Schulz flops
    per_iter = work["gram"][1] + work["gram2_epilogue"][1] + work["x_update"][1]
    assert per_iter * w.ns_steps == w.ns_flops()


def test_phase_work_fused_class_counts_every_iteration():
    w = W.WORKLOADS[4]                        # ragged: both classes present
    work = bench.phase_work(w, _ClassOf)
    assert work["ns_fused"][1] > 0 and work["gram"][1] > 0
    tiled = work["gram"][1] + work["gram2_epilogue"][1] + work["x_update"][1]
    assert tiled * w.ns_steps + work["ns_fused"][1] == w.ns_flops()


@pytest.mark.timeout(120)
def test_cpu_baseline_leg_on_a_small_sample():
    w = W.WORKLOADS[1]                        # one 256 x 768 fp32 matrix
    out = bench.cpu_baseline(w, target_s=0.01)
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s"
    assert out["value"] > 0 and out["cores"] >= 1 and out["seconds"] > 0
    assert "256x768" in out["sample"]


def test_issued_work_of_the_symmetric_kernels():
    """Upper-triangle tiles only: at m = 4096 with 256-tiles, 136 of the 256
    tiles of the Gram and C products are issued (t (t + 1) / 2, t = 16); the X
    update issues its full padded product."""
    import bench
    import matrix_aware_optimizer_libmuon_amd as muon
    from matrix_aware_optimizer_libmuon_amd import workloads as W
    w = W.WORKLOADS[3]
    issued = bench.phase_issued(w, muon)
    work = bench.phase_work(w, muon)
    assert issued["gram"] / work["gram"][1] == pytest.approx(136 / 256)
    assert issued["gram2_epilogue"] / work["gram2_epilogue"][1] == pytest.approx(136 / 256)
    assert issued["x_update"] == work["x_update"][1]
