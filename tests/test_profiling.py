"""The bench's HBM-traffic figure comes from a committed counter profile and
is dropped (null) as soon as the kernel sources differ from the ones it was
measured on."""
import json

from matrix_aware_optimizer_libmuon_amd import profiling


def _profile(tmp_path, digest, value, phase="x_update"):
    p = tmp_path / "traffic.md"
    p.write_text("# t\n\n```json\n" + json.dumps(
        {"kernel_sources_sha256_16": digest, "traffic_bytes_per_launch": {phase: value}}) + "\n```\n")
    return str(p)


def test_traffic_is_reported_only_for_the_profiled_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(profiling, "TRAFFIC_PROFILE", _profile(tmp_path, profiling.kernel_sources_hash(), 123))
    assert profiling.current_traffic("x_update") == 123.0
    assert profiling.current_traffic("gram") is None
    monkeypatch.setattr(profiling, "TRAFFIC_PROFILE", _profile(tmp_path, "0" * 16, 123))
    assert profiling.current_traffic("x_update") is None
    monkeypatch.setattr(profiling, "TRAFFIC_PROFILE", str(tmp_path / "missing.md"))
    assert profiling.current_traffic("x_update") is None


def test_hash_covers_every_kernel_source():
    import os
    csrc = os.path.join(profiling.PKG, "csrc")
    kernels = {f for f in os.listdir(csrc) if f.endswith((".hip", ".h"))}
    assert kernels == set(profiling.KERNEL_SOURCES)


def _counters(path, counter, rows):
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (k, v) in enumerate(rows):
            f.write(f"{i},{k},{counter},{v}\n")
    return str(path)


def test_traffic_calibrates_on_the_largest_copy(tmp_path):
    # small descriptor uploads beside the 4 GiB calibration copy must not
    # dilute the factors; kernels are averaged over their dispatches
    copy = "__amd_rocclr_copyBuffer"
    f = _counters(tmp_path / "f.csv", "FETCH_SIZE",
                  [(copy, 1.0), (copy, 2 * 1024 * 1024.0), (copy, 3.0), ("muon::k_apply(int)", 10.0),
                   ("muon::k_apply(int)", 30.0)])
    w = _counters(tmp_path / "w.csv", "WRITE_SIZE",
                  [(copy, 4 * 1024 * 1024.0), (copy, 5.0), ("muon::k_apply(int)", 40.0)])
    text = profiling.traffic_summary(f, w, "t", "cmd")
    assert "factors are 2.000 (fetch) and 1.000 (write)" in text
    data = json.loads(text.split("```json\n")[1].split("\n```")[0])
    assert data["traffic_bytes_per_launch"]["apply"] == round((20.0 * 2 + 40.0) * 1024)


def test_per_kernel_stamps(tmp_path, monkeypatch):
    # a kernel's figure survives changes to sources it is not built from
    stamps = {"x_update": profiling.kernel_sources_hash("x_update")}
    monkeypatch.setattr(profiling, "TRAFFIC_PROFILE", _profile(tmp_path, stamps, 7))
    assert profiling.current_traffic("x_update") == 7.0
    assert "muon_fused.hip" not in profiling.SOURCES_OF["x_update"]
    assert "muon_gemm.h" in profiling.SOURCES_OF["x_update"]
    monkeypatch.setattr(profiling, "TRAFFIC_PROFILE", _profile(tmp_path, {"x_update": "0" * 16}, 7))
    assert profiling.current_traffic("x_update") is None


def test_kernel_names_are_shortened_past_anonymous_namespaces():
    from matrix_aware_optimizer_libmuon_amd.profiling import _short
    assert _short("void muon::(anonymous namespace)::k_ns_fused<64>(muon::MatDesc const*, "
                  "float const*, int, int)") == "k_ns_fused<64>"
    assert _short("void muon::k_gram<256>(muon::MatDesc const*, long const*, int, long, int)") \
        == "k_gram<256>"


def test_telemetry_summary_reads_the_last_json_line(tmp_path):
    tele = {"samples": 10, "busy_samples": 9, "period_ms": 50.0, "power_cap_w": 1400.0,
            "power_w": {"median": 1360.0, "p10": 1300.0, "p90": 1370.0, "max": 1380.0},
            "power_median_frac_of_cap": 1360.0 / 1400.0,
            "gfxclk_mhz": {"median": 1800.0, "p10": 1750.0, "p90": 1900.0},
            "bf16_peak_at_median_clock_tflops": 1875.0, "roofline_kernel_frac_of_clock_peak": 0.66}
    line = {"ms_per_step": 505.0, "telemetry": tele,
            "roofline": {"kernel": "x_update", "achieved": 1237.5, "unit": "TFLOP/s", "frac": 0.495}}
    p = tmp_path / "bench.json"
    p.write_text("noise\n" + json.dumps(line) + "\n")
    text = profiling.telemetry_summary(str(p), "T", "python3 bench.py")
    assert text.startswith("# T\n") and "python3 bench.py" in text
    assert "| 1360 / 1300 / 1370 / 1380 W |" in text and "| 1400 W |" in text
    assert "1800 / 1750 / 1900 MHz" in text and "(9 of 10)" in text
    assert "0.495 of the quoted peak, 0.660 of the peak at the median clock" in text
    assert json.loads(text.split("```json\n")[1].split("\n```")[0]) == tele
