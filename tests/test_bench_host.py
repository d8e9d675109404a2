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


def test_telemetry_summary():
    """Medians and percentiles over the samples; entries the board reports as
    'N/A' (or not at all) are left out; the peak at the median clock scales
    the quoted bf16 peak by median clock / 2400 MHz."""
    samples = [{"power_w": p, "gfxclk_mhz": c, "xcd_gfxclk_mhz": [c - 10, c + 10], "hotspot_c": t,
                "gfx_activity": 100}
               for p, c, t in [(1300, 1700, 50), (1350, 1750, 55), (1400, 1800, 58)]]
    samples.append({"power_w": "N/A", "gfxclk_mhz": None, "xcd_gfxclk_mhz": "N/A", "hotspot_c": "N/A",
                    "gfx_activity": 100})
    # an idle reading (the board's metrics lag the start of the run) is left out
    samples.append({"power_w": 260, "gfxclk_mhz": 177, "xcd_gfxclk_mhz": [177, 177], "hotspot_c": 45,
                    "gfx_activity": 0})
    t = bench.summarize_telemetry(samples, 1400.0, 0.05, min_busy=3)
    assert t["samples"] == 5 and t["busy_samples"] == 4 and t["period_ms"] == 50.0
    assert t["power_w"]["median"] == 1350 and t["power_w"]["max"] == 1400
    assert t["power_median_frac_of_cap"] == pytest.approx(1350 / 1400)
    assert t["gfxclk_mhz"]["median"] == 1750
    assert t["bf16_peak_at_median_clock_tflops"] == pytest.approx(2500.0 * 1750 / 2400)
    assert t["xcd_gfxclk_mhz_median"] == [1740.0, 1760.0]
    assert t["hotspot_c_max"] == 58
    # nothing numeric: only the bookkeeping keys
    t = bench.summarize_telemetry([{"power_w": "N/A", "gfx_activity": 100}], None, 0.05, min_busy=1)
    assert "power_w" not in t and "gfxclk_mhz" not in t and t["power_cap_w"] is None
    # too few busy samples (a short timed region): no figures, a note instead
    t = bench.summarize_telemetry(samples, 1400.0, 0.05)
    assert "note" in t and "power_w" not in t and "bf16_peak_at_median_clock_tflops" not in t


def test_telemetry_without_a_gpu_reports_an_error_and_restores_stdout(capfd):
    """Here (no GPU) the tooling cannot sample: stop() returns an error entry
    and standard output is back on its own file afterwards."""
    tele = bench.Telemetry()
    tele.start()
    os.write(1, b"while sampling\n")   # what a library would write to file 1: on stderr
    t = tele.stop()
    os.write(1, b"after\n")
    out, err = capfd.readouterr()
    assert "error" in t
    assert "after" in out and "while sampling" not in out and "while sampling" in err
