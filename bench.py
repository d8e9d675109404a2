"""Benchmark of the Muon step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3]

One step = one muon_step call over the whole workload (momentum + norm,
normalise + cast, 5 x {Gram, Gram^2 epilogue, X update}, apply), with every
input already resident in HBM.  Timing: W untimed warm-up steps, then K timed
steps, each bracketed by HIP events on the launch stream; before each step the
momentum and parameter buffers are restored from a device copy (outside the
events), so every repetition sees identical inputs.  The whole timed loop is
bracketed by device synchronisations; its wall time (restores included) is
reported too.  Prints ONE JSON line:

* value: nominal Newton-Schulz TFLOP/s of the whole step, counting
  4 m^2 n + 2 m^3 per iteration and matrix (m the short side) over the
  median step time;
* matrices_per_s, NS-only TFLOP/s, fractions of the bf16 dense MFMA peak;
* roofline: the dominant kernel's algorithmic work per launch over its
  average launch time (HIP events on the launch stream, inside the timed
  region) against its roofline;
* measured_ceiling: second denominators measured on this GPU (the
  platform's bf16 GEMM on the X-update products, a device copy);
* cpu_baseline: the fp64 oracle timed on a bounded sample of the same
  workload on this host;
* telemetry: board power and GFX clock sampled (read-only, amdsmi) on a side
  thread over the timed steps, the bf16 MFMA peak at that clock, and the
  dominant kernel's rate against it (--no-telemetry leaves it out).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Muon step NS TFLOP/s + matrices/s at 1 GPU; % of bf16 MFMA peak"
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
QUINTIC = (3.4445, -4.7750, 2.0315)
FUSED_TILE = 32                 # padding granule the library reports for the fused class
NS_PHASES = ("gram", "gram2_epilogue", "x_update", "ns_fused")
NOMINAL_CLOCK_MHZ = 2400.0      # the clock the MFMA peak is quoted at


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def phase_work(w, muon):
    """Algorithmic work of one launch of each phase over the workload:
    flops for the MFMA phases (per Newton-Schulz iteration: X X^T 2 m^2 n,
    A A 2 m^3, C X 2 m^2 n; the fused launch runs every iteration of the
    small matrices, the tiled ones one iteration of the others), HBM bytes
    for the elementwise ones (momentum: read G and M, write M; normalise:
    read M, write bf16 X0; apply: read p and bf16 O, write p)."""
    gram = gram2 = xupd = fused = 0
    b_mom = b_norm = b_apply = 0
    gsz = 2 if w.grad_dtype == "bf16" else 4
    cls = {}
    for r, c in w.shapes:
        if (r, c) not in cls:  # the kernel class depends on the shape alone
            cls[(r, c)] = muon.workspace_view([(r, c)], 0, w.ns_steps)["tile"]
        m, n = min(r, c), max(r, c)
        if cls[(r, c)] == FUSED_TILE:
            fused += w.ns_steps * (4 * m * m * n + 2 * m ** 3)
        else:
            gram += 2 * m * m * n
            gram2 += 2 * m ** 3
            xupd += 2 * m * m * n
        e = r * c
        b_mom += e * (gsz + 8)
        b_norm += e * (4 + 2)
        b_apply += e * (4 + 2 + 4)
    return {"momentum_norm": ("hbm", b_mom), "normalize_cast": ("hbm", b_norm),
            "gram": ("mfma", gram), "gram2_epilogue": ("mfma", gram2),
            "x_update": ("mfma", xupd), "apply": ("hbm", b_apply), "ns_fused": ("mfma", fused)}


def phase_issued(w, muon):
    """MFMA work the tiled kernels actually issue per launch (padded shapes):
    the symmetric phases compute only the upper-triangle tiles, t (t + 1) / 2
    of a t x t tile grid, each 2 T^2 K flops; the X update every tile of the
    padded matrix, twice where C is a hi/lo pair."""
    gram = gram2 = xupd = 0
    for r, c in w.shapes:
        v = muon.workspace_view([(r, c)], 0, w.ns_steps)
        t = v["tile"]
        if t == FUSED_TILE:
            continue
        mp, npad = v["m_pad"], (v["rows_pad"] if v["transposed"] else v["cols_pad"])
        k = mp // t
        gram += k * (k + 1) // 2 * 2 * t * t * npad
        gram2 += k * (k + 1) // 2 * 2 * t * t * mp
        xupd += (2 if min(r, c) <= 128 else 1) * 2 * mp * mp * npad
    return {"gram": gram, "gram2_epilogue": gram2, "x_update": xupd}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, target_s: float = 20.0):
    """The fp64 oracle on a bounded sample of the workload's matrices, timed
    on this host's cores.  Returns the dict of the JSON line."""
    from oracle import muon_oracle as O
    from matrix_aware_optimizer_libmuon_amd import workloads as W
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    # sample: distinct shapes in workload order, smallest first, until the
    # estimated fp64 work would exceed the time target (>= 1 matrix)
    seen, order = set(), []
    for i, s in enumerate(w.shapes):
        if s not in seen:
            seen.add(s)
            order.append(i)
    order.sort(key=lambda i: w.shapes[i][0] * w.shapes[i][1])
    flops = 0
    done = []
    for idx in order:
        mi = W.matrix_inputs(w, idx)          # input generation is not timed
        r, c = w.shapes[idx]
        m, n = min(r, c), max(r, c)
        ts = time.perf_counter()
        O.muon_step_matrix(mi.param, mi.grad, mi.mom, lr=w.lr, mu=w.mu, wd=w.wd,
                           ns_steps=w.ns_steps, eps=w.eps, rms_mode=w.rms_mode)
        done.append((idx, time.perf_counter() - ts))
        flops += w.ns_steps * (4 * m * m * n + 2 * m ** 3)
        if sum(t for _, t in done) > target_s:
            break
    secs = sum(t for _, t in done)
    shapes = [f"{w.shapes[i][0]}x{w.shapes[i][1]}" for i, _ in done]
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus_visible": len(os.sched_getaffinity(0)),
            "seconds": secs, "matrices_per_s": len(done) / secs,
            "sample": f"{len(done)} matrices of the workload ({', '.join(shapes)}), one fp64 oracle "
                      f"step each (numpy, BLAS threads={cores}); input generation excluded"}


def measured_ceilings(torch, muon, w, dev, reps: int = 10):
    """Second denominators, measured on this GPU: the platform's bf16 GEMM
    (torch.matmul, i.e. hipBLASLt, as a black box) on the X-update products
    of the workload's tiled matrices, weighted like the launch (the faster of
    its NN and NT forms for the tall product, since C is symmetric), and a
    plain device copy for HBM."""
    shapes = {}
    for r, c in w.shapes:
        if muon.workspace_view([(r, c)], 0, w.ns_steps)["tile"] == FUSED_TILE:
            continue
        shapes[(r, c)] = shapes.get((r, c), 0) + 1
    out = {}

    def timed(f):
        for _ in range(3):
            f()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            f()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) / reps / 1e3

    if shapes:
        flops = secs = 0.0
        per = {}
        for (r, c), count in shapes.items():
            m, n = min(r, c), max(r, c)
            cm = torch.randn(m, m, device=dev).to(torch.bfloat16)
            cm = ((cm + cm.t()) * 0.5).contiguous()
            if r <= c:                       # X' = C X, X stored m x n
                x = torch.randn(m, n, device=dev).to(torch.bfloat16)
                o = torch.empty(m, n, device=dev, dtype=torch.bfloat16)
                t = timed(lambda: torch.matmul(cm, x, out=o))
            else:                            # X'^T = X^T C, stored n x m
                x = torch.randn(n, m, device=dev).to(torch.bfloat16)
                o = torch.empty(n, m, device=dev, dtype=torch.bfloat16)
                t = min(timed(lambda: torch.matmul(x, cm, out=o)),
                        timed(lambda: torch.matmul(x, cm.t(), out=o)))
            del cm, x, o
            per[f"{r}x{c}"] = 2 * m * m * n / t / 1e12
            flops += count * 2 * m * m * n
            secs += count * t
        out["x_update_vendor_gemm_tflops"] = flops / secs / 1e12
        out["vendor_gemm_tflops_by_shape"] = per
    n = 2**29                                # 2 GiB of fp32
    a = torch.ones(n, device=dev)
    b = torch.empty_like(a)
    t = timed(lambda: b.copy_(a))
    out["hbm_copy_gbs"] = 2 * 4 * n / t / 1e9
    del a, b
    out["method"] = ("torch.matmul (hipBLASLt) bf16 on the same products, one call per "
                     f"matrix, 3 warm-up + {reps} timed calls each (launch-bound for small "
                     "matrices, so there the fraction measures grouping as much as the "
                     "kernel); device copy of 2 GiB (read + write)")
    return out


def bench_adamw(torch, muon, dev, reps: int = 10):
    """AdamW branch on the parameters Muon does not take, for the d=4096
    transformer: token embedding and output head (32000 x 4096 each; the
    vocabulary size is a reading, the pages give none) and 65 norm weight
    vectors of 4096, bf16 gradients, fp32 params and moments; HBM-bound, 26
    algorithmic bytes per element (read p, g, m, v; write p, m, v)."""
    sizes = [32000 * 4096, 32000 * 4096] + [4096] * 65
    gen = torch.Generator(device=dev).manual_seed(7)
    p = [torch.randn(n, device=dev, generator=gen) * 0.02 for n in sizes]
    g = [(torch.randn(n, device=dev, generator=gen) * 1e-3).to(torch.bfloat16) for n in sizes]
    m = [torch.zeros(n, device=dev) for n in sizes]
    v = [torch.zeros(n, device=dev) for n in sizes]
    ws = muon.alloc_adamw_workspace(len(sizes), dev)
    steps = [1] * len(sizes)
    muon.adamw_step(p, g, m, v, steps, workspace=ws)
    torch.cuda.synchronize()
    muon.timing_enable(True)
    muon.timing_read()
    for r in range(reps):
        muon.adamw_step(p, g, m, v, [r + 2] * len(sizes), workspace=ws)
    t = muon.timing_read()["adamw"]
    muon.timing_enable(False)
    ms = t["ms"] / t["launches"]
    elements = sum(sizes)
    nbytes = elements * 26
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"workload": "embedding + head 32000x4096 each, 65 norm vectors of 4096; bf16 grads",
            "elements": elements, "avg_launch_ms": ms, "bound": "hbm", "achieved": gbs,
            "unit": "GB/s", "peak": HBM_PEAK_GBS, "frac": gbs / HBM_PEAK_GBS,
            "algorithmic_per_launch": nbytes}


def _num(v):
    return float(v) if isinstance(v, (int, float)) and not isinstance(v, bool) else None


def summarize_telemetry(samples, cap_w, period_s, min_busy=20):
    """Power and clock over the timed steps.  `samples`: dicts with power_w,
    gfxclk_mhz, xcd_gfxclk_mhz (one per XCD), hotspot_c and gfx_activity (%);
    entries the board does not report are None and are left out.  Only
    samples with the graphics engine at least half busy count (the board
    refreshes its metrics with a lag, so the first samples of a short run
    still show it idle); with fewer than `min_busy` of them the statistics
    are left out."""
    busy = [x for x in samples if (_num(x.get("gfx_activity")) or 0.0) >= 50.0]
    out = {"source": "amdsmi gpu metrics, read-only", "samples": len(samples),
           "busy_samples": len(busy), "period_ms": period_s * 1e3, "power_cap_w": cap_w}
    if len(busy) < min_busy:
        out["note"] = "too few samples with the GPU busy (timed region too short)"
        return out
    samples = busy
    pw = np.array([v for v in (_num(x.get("power_w")) for x in samples) if v is not None])
    ck = np.array([v for v in (_num(x.get("gfxclk_mhz")) for x in samples) if v is not None])
    if pw.size:
        out["power_w"] = {"median": float(np.median(pw)), "p10": float(np.percentile(pw, 10)),
                          "p90": float(np.percentile(pw, 90)), "max": float(pw.max())}
        if cap_w:
            out["power_median_frac_of_cap"] = float(np.median(pw)) / cap_w
    if ck.size:
        med = float(np.median(ck))
        out["gfxclk_mhz"] = {"median": med, "p10": float(np.percentile(ck, 10)),
                             "p90": float(np.percentile(ck, 90))}
        out["bf16_peak_at_median_clock_tflops"] = BF16_PEAK_TFLOPS * med / NOMINAL_CLOCK_MHZ
    xcd = [x.get("xcd_gfxclk_mhz") for x in samples]
    xcd = [r for r in xcd if isinstance(r, list) and r and all(_num(v) is not None for v in r)]
    if xcd and len({len(r) for r in xcd}) == 1:
        out["xcd_gfxclk_mhz_median"] = [float(v) for v in np.median(np.array(xcd, float), axis=0)]
    hot = [v for v in (_num(x.get("hotspot_c")) for x in samples) if v is not None]
    if hot:
        out["hotspot_c_max"] = max(hot)
    return out


class Telemetry:
    """Board power and GFX clock read from amdsmi on a side thread while the
    timed steps run.  Read-only queries; without the tooling (or a board that
    refuses them) the JSON line carries the error instead.  Standard output is
    pointed at standard error meanwhile, so that nothing the tooling prints can
    land beside the JSON line."""
    PERIOD_S = 0.05

    def __init__(self):
        self.samples, self.error, self.cap_w = [], None, None
        self._stop = threading.Event()
        self._th = None
        self._smi = None
        self._saved_stdout = None

    def start(self):
        sys.stdout.flush()
        self._saved_stdout = os.dup(1)
        os.dup2(2, 1)
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            cap = _num(amdsmi.amdsmi_get_power_cap_info(self._h).get("power_cap"))
            self.cap_w = cap / 1e6 if cap else None          # reported in microwatts
        except Exception as e:                                 # no tooling: no telemetry
            self.error = repr(e)
            return
        self._th = threading.Thread(target=self._run, daemon=True)
        self._th.start()

    def _run(self):
        while not self._stop.is_set():
            try:
                m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
            except Exception as e:
                self.error = repr(e)
                return
            self.samples.append({"power_w": m.get("current_socket_power"),
                                 "gfxclk_mhz": m.get("current_gfxclk"),
                                 "xcd_gfxclk_mhz": m.get("current_gfxclks"),
                                 "hotspot_c": m.get("temperature_hotspot"),
                                 "gfx_activity": m.get("average_gfx_activity")})
            self._stop.wait(self.PERIOD_S)

    def stop(self):
        if self._th is not None:
            self._stop.set()
            self._th.join()
        if self._smi is not None:
            try:
                self._smi.amdsmi_shut_down()
            except Exception:
                pass
        sys.stdout.flush()
        if self._saved_stdout is not None:
            os.dup2(self._saved_stdout, 1)
            os.close(self._saved_stdout)
            self._saved_stdout = None
        if not self.samples:
            return {"error": self.error or "no samples"}
        out = summarize_telemetry(self.samples, self.cap_w, self.PERIOD_S)
        if self.error:
            out["error"] = self.error
        return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-phase-timing", action="store_true")
    ap.add_argument("--no-adamw", action="store_true",
                    help="skip the AdamW-branch measurement (an extra object in the JSON line)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured second denominators (vendor GEMM, device copy)")
    ap.add_argument("--entry", choices=("eager", "plan", "noalloc"), default="eager",
                    help="entry point timed: muon_step (default), a prepared plan's step, or "
                         "muon_step_noalloc (workloads within its fixed scratch only)")
    ap.add_argument("--no-telemetry", action="store_true",
                    help="do not sample board power and clock over the timed steps")
    ap.add_argument("--copy-gib", type=float, default=0.0,
                    help="also run a plain device copy of this many GiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: it measures the Muon step on a single GPU "
              "(sharding across GPUs is described, not implemented); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import matrix_aware_optimizer_libmuon_amd as muon
    from matrix_aware_optimizer_libmuon_amd import workloads as W

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    muon._lib.load()          # fails loudly when libmuon.so is missing
    dev = torch.device("cuda:0")
    w = W.WORKLOADS[args.workload]
    log(f"[bench] workload {w.key}: {w.name}; {w.n_mats} matrices, {w.elements() / 1e9:.3f} G elements")

    t0 = time.perf_counter()
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 + w.key)
    params, grads, moms = [], [], []
    for i in range(w.n_mats):
        p, g, m = W.device_inputs(w, i, dev, gen)
        params.append(p)
        grads.append(g)
        moms.append(m)
    ws = muon.alloc_workspace(w.shapes, dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs on device in {time.perf_counter() - t0:.1f} s; workspace "
        f"{ws.numel() / 2**30:.2f} GiB; HBM in use {torch.cuda.memory_allocated() / 2**30:.1f} GiB")

    stream = torch.cuda.current_stream(dev)
    kw = dict(lr=w.lr, mu=w.mu, wd=w.wd, ns_steps=w.ns_steps, coeffs=QUINTIC,
              rms_scale=w.rms_mode, eps=w.eps, workspace=ws, stream=stream)
    if args.entry == "eager":
        def step():
            muon.muon_step(params, grads, moms, **kw)
    elif args.entry == "plan":
        plan = muon.Plan(params, grads, moms, **kw)

        def step():
            plan.step(stream)
    else:
        if muon.workspace_bytes(w.shapes) > muon.NOALLOC_SCRATCH_BYTES:
            print(f"workload {w.key} needs more workspace than muon_step_noalloc's fixed scratch",
                  file=sys.stderr)
            sys.exit(2)
        nkw = {k: v for k, v in kw.items() if k != "workspace"}

        def step():
            muon.muon_step_noalloc(params, grads, moms, **nkw)

    # device copies of the state the step updates, restored before every step
    p0 = [t.clone() for t in params]
    m0 = [t.clone() for t in moms]
    torch.cuda.synchronize()

    def restore():
        for t, src in zip(params, p0):
            t.copy_(src)
        for t, src in zip(moms, m0):
            t.copy_(src)

    for k in range(args.warmup):
        restore()
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup step {k + 1}/{args.warmup} done")

    if not args.no_phase_timing:
        muon.timing_enable(True)
        muon.timing_read()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    tele = None if args.no_telemetry else Telemetry()
    if tele is not None:
        tele.start()
    t_start = time.perf_counter()
    for k in range(args.steps):
        restore()
        ev[k][0].record(stream)
        step()
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    telemetry = tele.stop() if tele is not None else None
    phases = muon.timing_read() if not args.no_phase_timing else None
    muon.timing_enable(False)
    step_ms = np.array([a.elapsed_time(b) for a, b in ev])
    ms_per_step = float(np.median(step_ms))
    log(f"[bench] {args.steps} timed steps: median {ms_per_step:.3f} ms/step "
        f"(min {step_ms.min():.3f}, max {step_ms.max():.3f}; wall {elapsed * 1e3 / args.steps:.3f} "
        f"ms/step with the state restores)")
    del p0, m0

    flops_step = w.ns_flops()
    value = flops_step / (ms_per_step / 1e3) / 1e12
    out = {"metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded device draws of the workload's laws)",
           "config": {"workload": w.name, "n_matrices": w.n_mats, "entry": args.entry,
                      "shapes": sorted({f"{r}x{c}" for r, c in w.shapes}),
                      "grad_dtype": w.grad_dtype, "ns_steps": w.ns_steps,
                      "coeffs": list(QUINTIC), "lr": w.lr, "mu": w.mu, "wd": w.wd,
                      "eps": w.eps, "rms_scale": w.rms_mode},
           "matrices_per_s": w.n_mats / (ms_per_step / 1e3),
           "frac_of_bf16_peak": value / BF16_PEAK_TFLOPS,
           "nominal_ns_flops_per_step": flops_step,
           "timing": {"ms_per_step": "median of the per-step HIP-event times",
                      "step_ms_mean": float(step_ms.mean()), "step_ms_min": float(step_ms.min()),
                      "step_ms_max": float(step_ms.max()),
                      "wall_ms_per_step": elapsed * 1e3 / args.steps,
                      "between_steps": "momentum and parameters restored from a device copy"}}

    if phases is not None and any(r["launches"] for r in phases.values()):
        # (muon_step_noalloc records no phase timing: no events may be created)
        work = phase_work(w, muon)
        per = {}
        for name, rec in phases.items():
            n = rec["launches"]
            if n == 0:
                continue
            avg_ms = rec["ms"] / n
            kind, amount = work[name]
            if kind == "mfma":
                achieved = amount / (avg_ms / 1e3) / 1e12
                per[name] = {"launches_per_step": n / args.steps, "avg_launch_ms": avg_ms,
                             "bound": "mfma", "achieved": achieved, "unit": "TFLOP/s",
                             "peak": BF16_PEAK_TFLOPS, "frac": achieved / BF16_PEAK_TFLOPS,
                             "algorithmic_per_launch": amount}
            else:
                achieved = amount / (avg_ms / 1e3) / 1e9
                per[name] = {"launches_per_step": n / args.steps, "avg_launch_ms": avg_ms,
                             "bound": "hbm", "achieved": achieved, "unit": "GB/s",
                             "peak": HBM_PEAK_GBS, "frac": achieved / HBM_PEAK_GBS,
                             "algorithmic_per_launch": amount}
        # MFMA counters of the committed profile (null when the kernels
        # changed since it was taken), and the rate on the work the
        # symmetric kernels actually issue (upper-triangle tiles only)
        from matrix_aware_optimizer_libmuon_amd.profiling import current_mfma
        issued = phase_issued(w, muon)
        for name in ("gram", "gram2_epilogue", "x_update"):
            if name in per:
                busy, _ = current_mfma(name)
                per[name]["mfma_busy_per_cycle"] = busy
                per[name]["issued_per_launch"] = issued[name]
                per[name]["issued_frac"] = (issued[name] / (per[name]["avg_launch_ms"] / 1e3) / 1e12
                                            / BF16_PEAK_TFLOPS)
        ns_ms = sum(phases[k]["ms"] for k in NS_PHASES) / args.steps
        out["ns_ms_per_step"] = ns_ms
        out["ns_tflops"] = flops_step / (ns_ms / 1e3) / 1e12
        out["ns_frac_of_bf16_peak"] = out["ns_tflops"] / BF16_PEAK_TFLOPS
        out["phases"] = per
        # HBM bytes per launch from the committed rocprofv3 counter profile
        # (null when the kernels changed since it was taken)
        from matrix_aware_optimizer_libmuon_amd.profiling import current_traffic
        for name in per:
            per[name]["traffic"] = current_traffic(name)
        dom = max(per, key=lambda k: per[k]["avg_launch_ms"] * per[k]["launches_per_step"])
        d = per[dom]
        out["roofline"] = {"kernel": dom, "bound": d["bound"], "achieved": d["achieved"],
                           "peak": d["peak"], "unit": d["unit"], "frac": d["frac"],
                           "traffic": d["traffic"]}
        if "mfma_busy_per_cycle" in d:
            out["roofline"]["mfma_busy_per_cycle"] = d["mfma_busy_per_cycle"]
        if telemetry and d["bound"] == "mfma" and "bf16_peak_at_median_clock_tflops" in telemetry:
            telemetry["roofline_kernel_frac_of_clock_peak"] = (
                d["achieved"] / telemetry["bf16_peak_at_median_clock_tflops"])
    if telemetry is not None:
        out["telemetry"] = telemetry

    if args.copy_gib > 0:
        n = int(args.copy_gib * 2**30) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        log(f"[bench] copy calibration: {n * 4 / 2**30:.2f} GiB copied")

    if args.entry == "plan":
        del plan
    del params, grads, moms, ws
    torch.cuda.empty_cache()
    if not args.no_ceilings:
        ceil = measured_ceilings(torch, muon, w, dev)
        if "roofline" in out and out["roofline"]["kernel"] == "x_update" and \
                "x_update_vendor_gemm_tflops" in ceil:
            ceil["x_update_frac_of_vendor"] = (out["roofline"]["achieved"]
                                               / ceil["x_update_vendor_gemm_tflops"])
        out["measured_ceiling"] = ceil
        torch.cuda.empty_cache()
    if not args.no_adamw:
        out["adamw"] = bench_adamw(torch, muon, dev)
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 CPU oracle on a sample ...")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
