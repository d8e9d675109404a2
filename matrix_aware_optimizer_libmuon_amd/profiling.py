"""rocprofv3 summaries for profiles/ and the HBM-traffic figure of bench.py.

    python -m matrix_aware_optimizer_libmuon_amd.profiling trace  <kernel_stats.csv> <title> <command>
    python -m matrix_aware_optimizer_libmuon_amd.profiling traffic <fetch.csv> <write.csv> <title> <commands>

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
              "ns_fused": _COMMON + ("muon_fused.hip",)}
KERNEL_SOURCES = tuple(sorted({f for files in SOURCES_OF.values() for f in files}))
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "muon_step_transformer_d4096_hbm_traffic.md")

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


def current_traffic(phase: str):
    """HBM bytes per launch of `phase` from the committed profile, or None when
    there is none or the kernels changed since it was taken."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    data = json.loads(m.group(1))
    v = data.get("traffic_bytes_per_launch", {}).get(phase)
    if v is None or phase not in SOURCES_OF:
        return None
    stamp = data.get("kernel_sources_sha256_16")
    # per-kernel stamps; a single string stamps every kernel with all sources
    want = stamp.get(phase) if isinstance(stamp, dict) else stamp
    have = kernel_sources_hash(phase) if isinstance(stamp, dict) else kernel_sources_hash()
    return float(v) if want == have else None


if __name__ == "__main__":
    if sys.argv[1] == "trace":
        sys.stdout.write(trace_summary(sys.argv[2], sys.argv[3], sys.argv[4]))
    elif sys.argv[1] == "traffic":
        sys.stdout.write(traffic_summary(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5]))
    else:
        raise SystemExit(__doc__)
