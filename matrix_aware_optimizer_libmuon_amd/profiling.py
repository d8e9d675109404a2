"""rocprofv3 summaries for profiles/ and the HBM-traffic figure of bench.py.

    python -m matrix_aware_optimizer_libmuon_amd.profiling trace  <kernel_stats.csv> <title> <command>
    python -m matrix_aware_optimizer_libmuon_amd.profiling traffic <fetch.csv> <write.csv> <title> <commands>
    python -m matrix_aware_optimizer_libmuon_amd.profiling mfma <counters.csv> <kernel_trace.csv> <title> <command>
    python -m matrix_aware_optimizer_libmuon_amd.profiling counters <counters.csv> <title> <command>
    python -m matrix_aware_optimizer_libmuon_amd.profiling telemetry <bench.json> <title> <command>

The MFMA summary records, per Newton-Schulz GEMM kernel, the fraction of
cycles the MFMA units were busy (rocprofv3's MfmaUtil: SQ_VALU_MFMA_BUSY_CYCLES
over GRBM_GUI_ACTIVE times the SIMD count), the bf16 MFMA work issued
(SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 flops) and the shader clock the kernel
ran at, stamped like the traffic figures.

The traffic summary records, per libmuon kernel, FETCH_SIZE and WRITE_SIZE
(KiB per dispatch) scaled by what the same counters read for a plain device
copy of known size in the same run, and stamps each kernel's figure with a
hash of the sources that kernel is built from.  bench.py reports a kernel's
traffic only while that hash still matches the sources (a changed kernel
makes its figure stale: null).
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
_COMMON = ("muon_device.h", "muon_internal.h")
_ELEMENTWISE = _COMMON + ("muon_kernels.hip",)
_GEMM = _COMMON + ("muon_gemm.h", "muon_gemm256.hip", "muon_gemm128.hip")
# the sources each bench phase's kernel is compiled from
SOURCES_OF = {"momentum_norm": _ELEMENTWISE, "normalize_cast": _ELEMENTWISE, "apply": _ELEMENTWISE,
              "adamw": _ELEMENTWISE, "gram": _GEMM, "gram2_epilogue": _GEMM, "x_update": _GEMM,
              "ns_fused": _COMMON + ("muon_fused.hip",),
              # the descriptor-table writer of the no-allocation step (no bench phase)
              "noalloc_table": _COMMON + ("muon_noalloc.hip",)}
KERNEL_SOURCES = tuple(sorted({f for files in SOURCES_OF.values() for f in files}))
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "muon_step_transformer_d4096_hbm_traffic.md")
MFMA_PROFILE = os.path.join(ROOT, "profiles", "muon_step_transformer_d4096_mfma_util.md")

# kernel symbol -> bench phase name
PHASE_OF = {"k_momentum_norm": "momentum_norm", "k_normalize": "normalize_cast",
            "k_gram<256>": "gram", "k_gram2<256>": "gram2_epilogue",
            "k_xupdate<256>": "x_update", "k_apply": "apply"}


def kernel_sources_hash(phase: str | None = None) -> str:
    """sha256[:16] over the sources of `phase` (all kernel sources if None)."""
    h = hashlib.sha256()
    for name in (SOURCES_OF[phase] if phase else KERNEL_SOURCES):
        with open(os.path.join(PKG, "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    """Kernel name without return type, namespaces and argument list."""
    name = name.replace("(anonymous namespace)::", "")
    name = re.sub(r"^void\s+", "", name.split("(")[0])
    return name.replace("muon::", "")


def trace_summary(stats_csv: str, title: str, command: str) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    out = [f"# {title}", "", "Command (repository root, one MI355X):", "", "```", command, "```", "",
           "| kernel | calls | total ms | avg ms | % of GPU time |", "|---|---:|---:|---:|---:|"]
    for r in rows:
        out.append(f"| `{_short(r['Name'])[:70]}` | {int(r['Calls'])} | "
                   f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['AverageNs']) / 1e6:.4f} | "
                   f"{float(r['Percentage']):.2f} |")
    return "\n".join(out) + "\n"


def _per_kernel(csv_path: str, reduce=None) -> dict:
    acc = defaultdict(list)
    for r in csv.DictReader(open(csv_path)):
        acc[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: (reduce(v) if reduce else sum(v) / len(v)) for k, v in acc.items()}


def traffic_summary(fetch_csv: str, write_csv: str, title: str, commands: str,
                    copy_bytes: int = 4 << 30) -> str:
    fetch, write = _per_kernel(fetch_csv), _per_kernel(write_csv)
    copy = "__amd_rocclr_copyBuffer"
    # the calibration copy is the largest copy dispatch of the run (small
    # ones are descriptor uploads)
    fetch[copy] = _per_kernel(fetch_csv, max)[copy]
    write[copy] = _per_kernel(write_csv, max)[copy]
    f_scale = copy_bytes / (fetch[copy] * 1024.0)
    w_scale = copy_bytes / (write[copy] * 1024.0)
    out = [f"# {title}", "", "Commands (repository root, one MI355X; one counter per run):", "", "```",
           commands, "```", "",
           f"Calibration: a plain copy of {copy_bytes / 2**30:.0f} GiB (`{copy}`, same run) reads "
           f"{fetch[copy]:.4g} KiB on FETCH_SIZE and {write[copy]:.4g} KiB on WRITE_SIZE, so the factors "
           f"are {f_scale:.3f} (fetch) and {w_scale:.3f} (write).", "",
           "| kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | HBM bytes/dispatch (scaled) |",
           "|---|---:|---:|---:|"]
    traffic = {}
    for sym, phase in PHASE_OF.items():
        if sym in fetch and sym in write:
            b = fetch[sym] * 1024.0 * f_scale + write[sym] * 1024.0 * w_scale
            traffic[phase] = b
            out.append(f"| `{sym}` | {fetch[sym]:.4g} | {write[sym]:.4g} | {b:.4g} |")
    out += ["", "Machine-readable (bench.py reports a kernel's traffic only while the hash matches "
            "the kernel sources):", "", "```json",
            json.dumps({"kernel_sources_sha256_16": {k: kernel_sources_hash(k) for k in traffic},
                        "traffic_bytes_per_launch": {k: round(v) for k, v in traffic.items()}}),
            "```"]
    return "\n".join(out) + "\n"


def mfma_summary(counters_csv: str, trace_csv: str, title: str, command: str) -> str:
    """Per GEMM kernel: mean MfmaUtil (busy fraction), issued bf16 MFMA flops
    per dispatch, GRBM_GUI_ACTIVE per dispatch (summed over the 8 XCDs by the
    profiler, so divided by 8 here) and the clock that implies over the
    kernel-trace duration of the same dispatches."""
    util = _per_kernel_counter(counters_csv, "MfmaUtil")
    mops = _per_kernel_counter(counters_csv, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    gui = _per_kernel_counter(counters_csv, "GRBM_GUI_ACTIVE")
    dur = defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        dur[_short(r["Kernel_Name"])].append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    out = [f"# {title}", "", "Command (repository root, one MI355X; counters in their own run):", "",
           "```", command, "```", "",
           "MfmaUtil is rocprofv3's derived metric: SQ_VALU_MFMA_BUSY_CYCLES summed over every SIMD, "
           "over GRBM_GUI_ACTIVE (max over XCDs) times the SIMD count (1024). Issued flops are "
           "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512. The clock is GRBM_GUI_ACTIVE per XCD over the "
           "dispatch's duration in the same run.", "",
           "| kernel | MFMA busy / cycle | issued bf16 TFLOP / dispatch | GPU cycles / dispatch | "
           "duration ms (profiled) | clock GHz |", "|---|---:|---:|---:|---:|---:|"]
    busy, issued = {}, {}
    for sym, phase in PHASE_OF.items():
        if sym not in util or phase not in ("gram", "gram2_epilogue", "x_update"):
            continue
        cyc = gui.get(sym, 0.0) / 8.0
        ms = sum(dur[sym]) / len(dur[sym]) / 1e6 if dur.get(sym) else float("nan")
        ghz = cyc / (ms * 1e6) if ms == ms and ms > 0 else float("nan")
        busy[phase] = util[sym] / 100.0
        issued[phase] = mops.get(sym, 0.0) * 512
        out.append(f"| `{sym}` | {busy[phase]:.3f} | {issued[phase] / 1e12:.2f} | {cyc:.4g} | "
                   f"{ms:.3f} | {ghz:.2f} |")
    out += ["", "Machine-readable (bench.py reports a kernel's figure only while the hash matches "
            "the kernel sources):", "", "```json",
            json.dumps({"kernel_sources_sha256_16": {k: kernel_sources_hash(k) for k in busy},
                        "mfma_busy_per_cycle": {k: round(v, 4) for k, v in busy.items()},
                        "issued_bf16_flops_per_dispatch": {k: round(v) for k, v in issued.items()}}),
            "```"]
    return "\n".join(out) + "\n"


def telemetry_summary(bench_json: str, title: str, command: str) -> str:
    """Board power and GFX clock over bench.py's timed steps (its `telemetry`
    object), with the step time and the dominant kernel's rate beside them."""
    with open(bench_json) as f:
        d = json.loads(f.read().strip().splitlines()[-1])
    t, r = d.get("telemetry") or {}, d.get("roofline") or {}
    out = [f"# {title}", "", "Command (repository root, one MI355X):", "", "```", command, "```", "",
           "Sampled every {:.0f} ms from the board's metrics (read-only) over the timed steps; only "
           "samples with the graphics engine at least half busy count ({} of {}).".format(
               t.get("period_ms", float("nan")), t.get("busy_samples"), t.get("samples")), "",
           "| quantity | value |", "|---|---|",
           f"| step time (median) | {d.get('ms_per_step', float('nan')):.1f} ms |"]
    if "power_w" in t:
        p = t["power_w"]
        out.append(f"| board power: median / p10 / p90 / max | {p['median']:.0f} / {p['p10']:.0f} / "
                   f"{p['p90']:.0f} / {p['max']:.0f} W |")
    if t.get("power_cap_w"):
        out.append(f"| power cap | {t['power_cap_w']:.0f} W |")
    if "power_median_frac_of_cap" in t:
        out.append(f"| median power / cap | {t['power_median_frac_of_cap']:.3f} |")
    if "gfxclk_mhz" in t:
        c = t["gfxclk_mhz"]
        out.append(f"| GFX clock: median / p10 / p90 | {c['median']:.0f} / {c['p10']:.0f} / "
                   f"{c['p90']:.0f} MHz (2400 MHz nominal) |")
    if "xcd_gfxclk_mhz_median" in t:
        out.append("| per-XCD clock medians | " + ", ".join(f"{v:.0f}" for v in t["xcd_gfxclk_mhz_median"])
                   + " MHz |")
    if "hotspot_c_max" in t:
        out.append(f"| hotspot temperature, max | {t['hotspot_c_max']:.0f} C |")
    if "bf16_peak_at_median_clock_tflops" in t:
        out.append(f"| bf16 MFMA peak at the median clock | {t['bf16_peak_at_median_clock_tflops']:.0f} "
                   f"TFLOP/s |")
    if r:
        out.append(f"| dominant kernel (`{r.get('kernel')}`) | {r.get('achieved', float('nan')):.0f} "
                   f"{r.get('unit', '')}: {r.get('frac', float('nan')):.3f} of the quoted peak, "
                   f"{t.get('roofline_kernel_frac_of_clock_peak', float('nan')):.3f} of the peak at "
                   f"the median clock |")
    out += ["", "```json", json.dumps(t), "```"]
    return "\n".join(out) + "\n"


def counters_summary(counters_csv: str, title: str, command: str) -> str:
    """Mean value per dispatch of every counter in the run, for each libmuon
    kernel (rocprofv3 sums a counter over its hardware instances)."""
    rows = list(csv.DictReader(open(counters_csv)))
    names = sorted({r["Counter_Name"] for r in rows})
    kernels = [k for k in PHASE_OF if any(_short(r["Kernel_Name"]) == k for r in rows)]
    kernels += sorted({_short(r["Kernel_Name"]) for r in rows if _short(r["Kernel_Name"]).startswith(
        ("k_gram<128>", "k_gram2<128>", "k_xupdate<128>", "k_ns_fused"))} - set(kernels))
    vals = {n: _per_kernel_counter(counters_csv, n) for n in names}
    out = [f"# {title}", "", "Command (repository root, one MI355X; counters in their own run):", "",
           "```", command, "```", "",
           "Mean per dispatch. GRBM_GUI_ACTIVE is summed over the 8 XCDs (cycles per XCD = value / 8); "
           "MfmaUtil is a percentage of MFMA-busy SIMD cycles; SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 = bf16 "
           "flops issued; TCC_* count L2 requests, hits and misses over all channels.", "",
           "| kernel | " + " | ".join(names) + " |", "|---|" + "---:|" * len(names)]
    for k in kernels:
        out.append(f"| `{k}` | " + " | ".join(f"{vals[n].get(k, float('nan')):.4g}" for n in names) + " |")
    return "\n".join(out) + "\n"


def _per_kernel_counter(csv_path: str, counter: str) -> dict:
    acc = defaultdict(list)
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] == counter:
            acc[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def _stamped(path: str, key: str, phase: str):
    try:
        text = open(path).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    data = json.loads(m.group(1))
    v = data.get(key, {}).get(phase)
    if v is None or phase not in SOURCES_OF:
        return None
    stamp = data.get("kernel_sources_sha256_16")
    # per-kernel stamps; a single string stamps every kernel with all sources
    want = stamp.get(phase) if isinstance(stamp, dict) else stamp
    have = kernel_sources_hash(phase) if isinstance(stamp, dict) else kernel_sources_hash()
    return float(v) if want == have else None


def current_mfma(phase: str):
    """(MFMA busy per cycle, issued bf16 flops per dispatch) of `phase` from the
    committed counter profile; None entries when absent or stale."""
    return (_stamped(MFMA_PROFILE, "mfma_busy_per_cycle", phase),
            _stamped(MFMA_PROFILE, "issued_bf16_flops_per_dispatch", phase))


def current_traffic(phase: str):
    """HBM bytes per launch of `phase` from the committed profile, or None when
    there is none or the kernels changed since it was taken."""
    return _stamped(TRAFFIC_PROFILE, "traffic_bytes_per_launch", phase)


if __name__ == "__main__":
    if sys.argv[1] == "trace":
        sys.stdout.write(trace_summary(sys.argv[2], sys.argv[3], sys.argv[4]))
    elif sys.argv[1] == "traffic":
        sys.stdout.write(traffic_summary(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5]))
    elif sys.argv[1] == "counters":
        sys.stdout.write(counters_summary(sys.argv[2], sys.argv[3], sys.argv[4]))
    elif sys.argv[1] == "telemetry":
        sys.stdout.write(telemetry_summary(sys.argv[2], sys.argv[3], sys.argv[4]))
    elif sys.argv[1] == "mfma":
        sys.stdout.write(mfma_summary(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5]))
    else:
        raise SystemExit(__doc__)
