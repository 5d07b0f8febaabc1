"""Benchmark: fwd+bwd attention TFLOP/s and % of bf16 dense MFMA peak on one MI355X.

One step = fa_fwd -> fa_bwd_preprocess -> fa_bwd_dkv -> fa_bwd_dq on inputs
already resident in HBM (the whole hot path, through the C ABI). First a
clock-settle phase (back-to-back steps for --settle-ms of wall time: the
chip's clocks take some 50-100 ms of sustained work to come up), then W
untimed warm-up steps, then K timed steps bracketed by synchronisation; HIP
events on the stream the kernels are launched on give the step time and, in
a second timed pass, each kernel's average duration. The settle phase's
length is part of the printed line. After the timed passes the workload runs
back to back for another --clock-ms of wall time while a host thread samples
the GFX clock (amdsmi, when available; its reading is refreshed too slowly
for the short timed passes themselves), and the MFMA peak is also given at
that measured clock.

FLOP count (algorithmic): N = allowed (i, j) pairs per (batch, head), exactly
counted from the mask; forward = 4*D*N*B*Hq, backward = 2.5 x forward.
The "formula" count halves the dense count under causal masking and ignores
the window.

Prints ONE JSON line. --gpus N > 1 exits: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
METRIC = "fwd+bwd attention TFLOP/s and % of bf16 MFMA peak (1 GPU)"
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_digest() -> str:
    """sha256 over the library's sources and compile flags: HBM byte counts
    taken with rocprofv3 are reported only while this digest still matches."""
    import hashlib

    from attention_fa_fwd_06_amd import build as fa_build

    hsh = hashlib.sha256()
    for name in sorted(fa_build.SOURCES) + sorted(
            n for n in os.listdir(fa_build.CSRC) if n.endswith((".hpp", ".h"))):
        hsh.update(name.encode())
        with open(os.path.join(fa_build.CSRC, name), "rb") as fh:
            hsh.update(fh.read())
    hsh.update(repr((fa_build.ARCH, fa_build.COMMON)).encode())
    return hsh.hexdigest()


def measured_traffic(workload_name: str, kernel: str):
    """Calibrated HBM bytes per launch (FETCH_SIZE + WRITE_SIZE) of `kernel` on
    `workload_name` from the committed counter summary, or None when there is
    none or the kernels have changed since it was taken."""
    path = os.path.join(PROFILES, f"hbm_traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256") != kernel_source_digest():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else float(k["bytes_per_launch"])


def allowed_pairs(Lq: int, Lkv: int, causal: bool, window: int) -> int:
    """Exact count of allowed (i, j) pairs under the mask rule."""
    total = 0
    for i in range(Lq):
        hi = min(i, Lkv - 1) if causal else Lkv - 1
        lo = max(0, i - window + 1) if window else 0
        if causal or not window:
            total += max(0, hi - lo + 1)
        else:  # window without causal: past trimmed, all future keys kept
            total += max(0, Lkv - lo)
    return total


def workload_flops(w):
    n = allowed_pairs(w.Lq, w.Lkv, w.causal, w.window)
    fwd = 4.0 * w.D * n * w.B * w.Hq
    dense = 4.0 * w.D * w.Lq * w.Lkv * w.B * w.Hq * (0.5 if w.causal else 1.0)
    return {"pairs": n, "fwd": fwd, "bwd": 2.5 * fwd, "total": 3.5 * fwd, "formula_total": 3.5 * dense,
            # per-kernel work actually required by each kernel's own outputs:
            # dK/dV: S, dP, dV, dK = 4 contractions; dQ: S, dP, dQ = 3
            "dkv": 8.0 * w.D * n * w.B * w.Hq, "dq": 6.0 * w.D * n * w.B * w.Hq}


def workload_bytes(w):
    e = {"f32": 4, "f16": 2, "bf16": 2}[w.dtype]
    q = w.B * w.Hq * w.Lq * w.D * e
    kv = w.B * w.Hkv * w.Lkv * w.D * e
    row = w.B * w.Hq * w.Lq * 4
    return {"fwd": 2 * q + 2 * kv + row, "pre": 2 * q + row, "dkv": 2 * q + 4 * kv + 2 * row,
            "dq": 3 * q + 2 * kv + 2 * row}


class ClockSampler:
    """Samples the GPU's GFX clock (MHz) from a host thread through amdsmi while
    started; `summary()` is None when amdsmi is unavailable or gives no
    reading."""

    def __init__(self):
        self.samples, self.error, self._h, self._stop, self._thr = [], None, None, None, None
        try:
            import amdsmi
            import torch

            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            if len(handles) == 1:
                self._h = handles[0]
            else:  # match the PCI bus of HIP device 0
                bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
                for h in handles:
                    bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)
                    if bus is not None and int(bdf.split(":")[1], 16) == int(bus):
                        self._h = h
            if self._h is None:
                self.error = "no amdsmi handle for HIP device 0"
            self._smi = amdsmi
        except Exception as e:  # pragma: no cover - depends on the box
            self.error = f"amdsmi unavailable: {type(e).__name__}"

    def _read(self):
        info = self._smi.amdsmi_get_clock_info(self._h, self._smi.AmdSmiClkType.GFX)
        return float(info["clk"])

    def start(self):
        if self._h is None:
            return
        import threading

        self._stop = threading.Event()

        def loop():
            while not self._stop.is_set():
                try:
                    self.samples.append(self._read())
                except Exception as e:  # pragma: no cover
                    self.error = f"amdsmi read failed: {type(e).__name__}"
                    return
                self._stop.wait(0.002)

        self._thr = threading.Thread(target=loop, daemon=True)
        self._thr.start()

    def stop(self):
        if self._thr is not None:
            self._stop.set()
            self._thr.join()
            self._thr = None

    def summary(self):
        x = [c for c in self.samples if c >= 100.0]  # a reading of 0 is no reading
        if not x:
            return None
        return {"mean": round(sum(x) / len(x), 1), "min": min(x), "max": max(x), "samples": len(x)}


def time_gpu(w, steps: int, warmup: int, settle_ms: float = 300.0, clock: ClockSampler | None = None,
             clock_ms: float = 1000.0):
    import torch

    import attention_fa_fwd_06_amd as fa
    from synth import to_torch, workload_inputs

    fa.load_library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    x = workload_inputs(w)
    q, k, v, do = (to_torch(x[n], w.dtype).to(dev) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    lse = torch.empty((w.B, w.Hq, w.Lq), device=dev, dtype=torch.float32)
    delta = torch.empty_like(lse)
    sc, ca, wi = w.scale, w.causal, w.window

    kernels = [
        ("fa_fwd", lambda: fa.fa_fwd(q, k, v, o, lse, sc, ca, wi)),
        ("fa_bwd_preprocess", lambda: fa.fa_bwd_preprocess(o, do, delta)),
        ("fa_bwd_dkv", lambda: fa.fa_bwd_dkv(q, k, v, do, lse, delta, dk, dv, sc, ca, wi)),
        ("fa_bwd_dq", lambda: fa.fa_bwd_dq(q, k, v, do, lse, delta, dq, sc, ca, wi)),
    ]

    def step():
        for _, f in kernels:
            f()

    # Clock settle: back-to-back steps until settle_ms of wall time has passed.
    # Each batch between synchronizations holds about 20 ms of GPU work (sized
    # from the batches before it), so that the queue never runs dry while the
    # host enqueues the next one.
    torch.cuda.synchronize()
    s0, n_settle, batch = time.perf_counter(), 0, 4
    while (time.perf_counter() - s0) * 1e3 < settle_ms:
        b0 = time.perf_counter()
        for _ in range(batch):
            step()
        torch.cuda.synchronize()
        n_settle += batch
        per_step = (time.perf_counter() - b0) / batch
        batch = max(4, min(10000, int(0.02 / max(per_step, 1e-6))))
    settle = {"ms": round((time.perf_counter() - s0) * 1e3, 1), "steps": n_settle}

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / steps

    # second pass: per-kernel durations, events around every launch
    ev = {name: [] for name, _ in kernels}
    for _ in range(steps):
        for name, f in kernels:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            f()
            b.record(stream)
            ev[name].append((a, b))
    torch.cuda.synchronize()
    per = {name: sum(a.elapsed_time(b) for a, b in pairs) / len(pairs) for name, pairs in ev.items()}

    # clock under sustained load of this workload (not part of any timing)
    if clock is not None and clock_ms > 0:
        batch = max(4, min(10000, int(20.0 / max(ms_step, 1e-3))))  # about 20 ms of GPU work per batch
        clock.samples = []
        clock.start()
        c0 = time.perf_counter()
        while (time.perf_counter() - c0) * 1e3 < clock_ms:
            for _ in range(batch):
                step()
            torch.cuda.synchronize()
        clock.stop()
    return ms_step, wall * 1e3 / steps, per, settle


def cpu_baseline(w, budget_s: float = 12.0, max_workers: int = 16):
    """The float64 oracle (oracle.backward as it stands) on a bounded sample of
    the workload, on the host's cores.

    The unit of work is one (batch, kv-group) slice: the full forward and
    backward of the group's query heads against its K and V. Slices run in a
    thread pool of one worker per available core (at most max_workers, BLAS
    held to one thread per worker), in waves of one slice per worker, until
    about budget_s of wall time has been spent. When a whole slice would take
    longer than about half the budget on one core (the 8192- and 32768-token
    workloads), each slice is cut to its first n query rows and keys (n at
    least twice the window, when there is one): under a
    causal mask those rows attend only to those keys, so the cut slice is a
    smaller instance of the same problem, and its work is counted exactly.
    Reported in TFLOP/s on the same algorithmic count as the GPU figure."""
    import concurrent.futures as cf

    from threadpoolctl import threadpool_limits

    import oracle
    from synth import decode, workload_inputs

    cores = max(1, min(max_workers, len(os.sched_getaffinity(0))))
    reps = w.Hq // w.Hkv
    # the oracle materialises every score: about 12 D FLOP per (row, key, head)
    # at roughly 1e10 FLOP/s on one core
    # (a cut slice keeps at least twice the window, so the window still trims it)
    n, n_min = w.Lq, max(64, min(w.Lq, 2 * w.window))
    while n // 2 >= n_min and 12.0 * n * n * w.D * reps / 1e10 > budget_s / 2:
        n //= 2
    cut = n < w.Lq
    Lq, Lkv = (n, min(n, w.Lkv)) if cut else (w.Lq, w.Lkv)
    x = workload_inputs(w)
    pairs = allowed_pairs(Lq, Lkv, w.causal, w.window)
    per_slice = 3.5 * 4.0 * w.D * pairs * reps

    def one(bg):
        b, g = bg
        hs = slice(g * reps, (g + 1) * reps)
        args = [decode(x["q"][b:b + 1, hs, :Lq], w.dtype), decode(x["k"][b:b + 1, g:g + 1, :Lkv], w.dtype),
                decode(x["v"][b:b + 1, g:g + 1, :Lkv], w.dtype), decode(x["do"][b:b + 1, hs, :Lq], w.dtype)]
        oracle.backward(*args, w.scale, w.causal, w.window)

    groups = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    done, t0 = 0, time.perf_counter()
    with threadpool_limits(limits=1, user_api="blas"), cf.ThreadPoolExecutor(cores) as ex:
        while done < len(groups) and time.perf_counter() - t0 < budget_s:
            wave = groups[done:done + cores]
            list(ex.map(one, wave))
            done += len(wave)
    secs = time.perf_counter() - t0
    what = f"first {Lq} query rows and {Lkv} keys of " if cut else ""
    return {"value": done * per_slice / secs / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{what}{done} of {len(groups)} (batch, kv-group) slices ({done * reps} of {w.B * w.Hq} "
                      f"query heads), full fwd+bwd in float64, {cores} threads, {secs:.2f} s",
            "seconds": secs}


def roofline(kernel: str, flops: float, nbytes: float, ms: float, peak_tflops: float) -> dict:
    """Roofline entry of one kernel: bound by the matrix cores when its
    algorithmic FLOP per byte is above the machine balance (peak FLOP/s over
    peak HBM bytes/s), else by HBM; achieved = algorithmic work / duration."""
    if flops / nbytes >= peak_tflops * 1e12 / (PEAK_HBM_GBS * 1e9):
        achieved = flops / (ms * 1e-3) / 1e12
        return {"kernel": kernel, "bound": "mfma", "achieved": achieved, "peak": peak_tflops, "unit": "TFLOP/s",
                "frac": achieved / peak_tflops}
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS}


def _r4(d):
    return {k: (round(v, 4) if isinstance(v, float) else v) for k, v in d.items()}


def _cpu_line(cb):
    cb = dict(cb)
    cb["value"] = float(f"{cb['value']:.4g}")
    cb["seconds"] = round(cb["seconds"], 2)
    return cb


def run(w, steps, warmup, settle_ms, cpu_budget, clock, clock_ms=1000.0):
    f = workload_flops(w)
    by = workload_bytes(w)
    ms, wall_ms, per, settle = time_gpu(w, steps, warmup, settle_ms, clock, clock_ms)
    tflops = f["total"] / (ms * 1e-3) / 1e12
    peak = PEAK_FP32_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS
    clk = clock.summary() if clock is not None else None
    res = {
        "workload": w,
        "ms_per_step": ms,
        "wall_ms_per_step": wall_ms,
        "tflops": tflops,
        "tflops_formula": f["formula_total"] / (ms * 1e-3) / 1e12,
        "pct_peak": 100.0 * tflops / peak,
        "per_kernel_ms": per,
        "fwd_ms": per["fa_fwd"],
        "bwd_ms": per["fa_bwd_preprocess"] + per["fa_bwd_dkv"] + per["fa_bwd_dq"],
        "flops": f,
        "bytes": by,
        "settle": settle,
        "clock": clk,
    }
    unit_flops = {"fa_fwd": f["fwd"], "fa_bwd_dkv": f["dkv"], "fa_bwd_dq": f["dq"]}
    unit_bytes = {"fa_fwd": by["fwd"], "fa_bwd_dkv": by["dkv"], "fa_bwd_dq": by["dq"]}
    # one roofline entry per MFMA kernel; the line's `roofline` is the dominant one
    res["kernels"] = {}
    for n in ("fa_fwd", "fa_bwd_dkv", "fa_bwd_dq"):
        e = roofline(n, unit_flops[n], unit_bytes[n], per[n], peak)
        e.update({"traffic": measured_traffic(w.name, n), "algorithmic_bytes": unit_bytes[n], "avg_ms": per[n]})
        if clk is not None and e["bound"] == "mfma":
            e["frac_at_measured_clock"] = e["achieved"] / (peak * clk["mean"] / 2400.0)
        res["kernels"][n] = e
    dom = max(("fa_fwd", "fa_bwd_dkv", "fa_bwd_dq"), key=lambda n: per[n])
    res["roofline"] = dict(res["kernels"][dom])
    res["roofline"]["traffic_unit"] = "HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE)"
    res["kernel_tflops"] = {n: unit_flops[n] / (per[n] * 1e-3) / 1e12 for n in unit_flops}
    res["pre_gbs"] = by["pre"] / (per["fa_bwd_preprocess"] * 1e-3) / 1e9
    if cpu_budget > 0:
        res["cpu_baseline"] = cpu_baseline(w, cpu_budget)
    return res


def _clock_fields(r, peak):
    clk = r["clock"]
    if clk is None:
        return {"gfx_clock_mhz": None, "peak_at_measured_clock": None, "pct_of_peak_at_measured_clock": None}
    # the published dense peak is 256 CUs x 4096 FLOP per clock at 2.4 GHz
    pk = peak * clk["mean"] / 2400.0
    return {"gfx_clock_mhz": clk, "peak_at_measured_clock": round(pk, 1),
            "pct_of_peak_at_measured_clock": round(100.0 * r["tflops"] / pk, 3)}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # The chip's clocks take some 50-100 ms of back-to-back steps to settle
    # (a 2048-token step runs 0.89 ms over its first 25 steps, 0.67 ms from
    # about step 75 on): the settle phase runs before the counted warm-up.
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="wall time of back-to-back steps run before the counted warm-up (clock settle)")
    ap.add_argument("--clock-ms", type=float, default=1000.0,
                    help="wall time of back-to-back steps, after the timed passes, over which the GFX clock is sampled")
    ap.add_argument("--workload", type=int, default=2, help="index into synth.WORKLOADS (default: the 2048-token GQA)")
    ap.add_argument("--also", type=str, default="0,1,3,4,5", help="comma list of extra workload indices reported inline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for the main workload")
    ap.add_argument("--also-cpu-budget", type=float, default=6.0, help="seconds of oracle time per extra workload")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain elementwise copy of MIB MiB (reference for HBM byte counters)")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this attention path runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    from synth import WORKLOADS

    if args.copy_calibration:
        import torch

        n = args.copy_calibration * (1 << 20) // 4
        x = torch.ones(n, device="cuda", dtype=torch.float32)
        y = torch.empty_like(x)
        for _ in range(3):
            torch.neg(x, out=y)  # reads and writes exactly MIB MiB each
        torch.cuda.synchronize()
        del x, y

    clock = ClockSampler()
    w = WORKLOADS[args.workload]
    cpu_main = 0.0 if args.no_cpu_baseline else args.cpu_budget
    cpu_also = 0.0 if args.no_cpu_baseline else args.also_cpu_budget
    main_res = run(w, args.steps, args.warmup, args.settle_ms, cpu_main, clock, args.clock_ms)
    extra = {}
    for idx in [int(s) for s in args.also.split(",") if s.strip() != ""]:
        if idx == args.workload:
            continue
        wx = WORKLOADS[idx]
        r = run(wx, args.steps, args.warmup, args.settle_ms, cpu_also, clock, args.clock_ms)
        wb = r["bytes"]
        extra[wx.name] = {
            "ms_per_step": round(r["ms_per_step"], 4), "tflops": round(r["tflops"], 2),
            # algorithmic HBM bytes of the four kernels over the step time (the
            # small cases are launch- and latency-bound, not MFMA-bound)
            "hbm_gbs": round((wb["fwd"] + wb["pre"] + wb["dkv"] + wb["dq"]) / (r["ms_per_step"] * 1e-3) / 1e9, 1),
            "tflops_formula": round(r["tflops_formula"], 2), "pct_peak": round(r["pct_peak"], 2),
            "per_kernel_ms": {k: round(v, 4) for k, v in r["per_kernel_ms"].items()},
            "roofline": _r4(r["roofline"]),
            "kernels": {k: _r4(v) for k, v in r["kernels"].items()},
            "clock_settle": r["settle"],
            **_clock_fields(r, PEAK_FP32_TFLOPS if wx.dtype == "f32" else PEAK_BF16_TFLOPS),
        }
        if "cpu_baseline" in r:
            extra[wx.name]["cpu_baseline"] = _cpu_line(r["cpu_baseline"])

    r = main_res
    peak = PEAK_FP32_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS
    line = {
        "metric": METRIC,
        "value": round(r["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle": r["settle"],
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs, the workload's shapes)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Lq": w.Lq, "Lkv": w.Lkv, "D": w.D,
                   "causal": w.causal, "window": w.window, "parallelism": "single GPU"},
        "pct_of_bf16_peak": round(r["pct_peak"], 3),
        **_clock_fields(r, peak),
        "tflops_formula_count": round(r["tflops_formula"], 3),
        "fwd_ms": round(r["fwd_ms"], 4),
        "bwd_ms": round(r["bwd_ms"], 4),
        "per_kernel_ms": {k: round(v, 4) for k, v in r["per_kernel_ms"].items()},
        "kernel_tflops": {k: round(v, 2) for k, v in r["kernel_tflops"].items()},
        "preprocess_gbs": round(r["pre_gbs"], 1),
        "roofline": _r4(r["roofline"]),
        "kernels": {k: _r4(v) for k, v in r["kernels"].items()},
        "cpu_baseline": _cpu_line(r["cpu_baseline"]) if "cpu_baseline" in r else None,
        "clock_sampler_error": clock.error,
        "also": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
