#!/usr/bin/env python3
"""Benchmark of C = A·Bᵀ on one MI355X through the libgemm_bt C-ABI.

One step = one gemm_bt call on the 4096×4096×4096 bf16 workload (A and B
i.i.d. N(0,1) rounded to bf16, seed 2, bf16 output), inputs resident in HBM.
Prints ONE JSON line on stdout:
  value        TFLOP/s of the whole job (2·M·N·K per step / wall time of the
               K timed steps between two synchronisations)
  timing       mean launch time of the timed steps (HIP events before and
               after them), the spread of a second pass with an event after
               every launch (median, min, max, p10, p90), and the untimed
               settle phase before them
  clock        the GPU clock (per-XCD gfxclk) and socket power of the first
               amdsmi metrics snapshot the firmware takes under continued
               launches of the workload after the timed steps (the table
               refreshes about once per second), and % of peak at that clock
  roofline     the tiled MFMA kernel against the MI355X dense bf16 peak;
               achieved = 2·M·N·K / the mean launch time
  cpu_baseline the CPU oracle timed on a bounded sample of the same product,
               with the host's CPU model and core counts
  secondary    the other workloads (1024×4096×4096 f16, 16×8192×8192
               skinny, 512³, 1000×3000×2050, 4096³ with E4M3 inputs against
               the fp8 peak, 4096³ int8 -> int32 against the int8 peak, a
               batch of 64 products of 512³ in one gemm_bt_batched call,
               4096³ with B stored K×N through gemm_bt_layout,
               1024×1024×16384, which gemm_bt_ws splits along K,
               1000×3000×2049, whose rows are only 2-byte aligned, and the
               thin 64×8192×8192, split along K on 64×64 tiles, against HBM
               bandwidth like the skinny product), timed the same way (us =
               mean launch time)
  copy_GBps    a plain 1 GiB device copy, as context for achievable HBM
Diagnostics go to stderr.  Whatever --warmup is, the timed steps follow an
untimed settle phase of at least 60 ms that then runs until the launch time
stops falling (bounded at 0.6 s): from idle the 4096³ launches take 124 us
and reach their steady 95-96 us only after 40-55 ms of sustained load.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-secondary]
  python bench.py --mode copy     # plain device copy of known size (counter calibration)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s and % of MI355X bf16 MFMA peak (4096³); µs @1024×4096×4096"
PEAK_BF16_TFLOPS = 2516.6  # 256 CU × 4096 dense bf16 FLOP/clk/CU × 2.4 GHz (published 2.5 PFLOP/s)
PEAK_FP8_TFLOPS = 5033.2   # twice the bf16 rate (published dense fp8: 5.0 PFLOP/s)
PEAK_I8_TOPS = 5033.2      # the same rate in integer operations (published dense int8: 5.0 POP/s)
PEAK_HBM_GBS = 8000.0      # published HBM3E bandwidth
MALL_BYTES = 256 << 20     # rotate inputs over more than the 256 MiB Infinity Cache


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_tiled_gemm_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they
    were taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(workload)
    if not ent or ent.get("kernel_source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


class ClockSampler:
    """amdsmi gpu_metrics snapshots on a background thread: (host time, firmware timestamp, per-XCD gfxclk MHz,
    socket W).  The firmware refreshes the table about once per second (measured on the MI355X boxes: one
    refresh in 1.5 s of polling), so a snapshot describes the GPU at its own refresh time, not at the time it
    is read.  Records nothing (and says why) when amdsmi is missing or refuses."""

    def __init__(self, period_s=0.002):
        self.samples = []
        self.error = None
        self.period = period_s
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi

            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            self.samples.append(self._read())
        except Exception as e:  # no amdsmi, no permission, no device: the bench still runs
            self.error = repr(e)

    def _read(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
        clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, int)]
        if not clks and isinstance(m.get("current_gfxclk"), int):
            clks = [m["current_gfxclk"]]
        pw = m.get("current_socket_power")
        fw = m.get("firmware_timestamp")
        return (time.perf_counter(), fw if isinstance(fw, int) else None, clks, pw if isinstance(pw, int) else None)

    def _loop(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._read())
            except Exception as e:
                self.error = repr(e)
                return
            time.sleep(self.period)

    def start(self):
        if self.error is None:
            self._thread = threading.Thread(target=self._loop, daemon=True)
            self._thread.start()
        return self

    def stop(self):
        self._stop.set()
        if self._thread:
            self._thread.join()

    def fresh_after(self, t):
        """The first snapshot the firmware took after host time t (its firmware timestamp differs from that
        of every sample read up to t), or None."""
        before = {x[1] for x in self.samples if x[0] <= t}
        for x in list(self.samples):
            if x[0] > t and x[1] not in before:
                return x
        return None


def clock_under_load(case, sampler, t_end, tflops, max_s=1.5):
    """The GPU clock under this workload: launches continue (untimed) after the timed steps until the
    firmware publishes a metrics snapshot taken after them, at most `max_s`; that snapshot's per-XCD gfxclk
    and socket power are reported, with the % of peak at the median clock."""
    if sampler.error is not None and not sampler.samples:
        return {"source": "amdsmi", "error": sampler.error}
    torch = case.torch
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    snap, n = None, 0
    while snap is None and time.perf_counter() - t0 < max_s:
        for i in range(20):
            case.step(n + i, stream.cuda_stream)
        n += 20
        stream.synchronize()
        snap = sampler.fresh_after(t_end)
    if snap is None:
        return {"source": "amdsmi", "error": "no fresh metrics snapshot within %.1f s of load" % max_s}
    clks = sorted(snap[2])
    med = clks[len(clks) // 2]
    peak_at = PEAK_BF16_TFLOPS * med / 2400.0  # 256 CU x 4096 FLOP/clk x sclk
    return {"source": "amdsmi gpu_metrics snapshot taken by the firmware under continued launches of the same "
                      "workload right after the timed steps (the table refreshes about once per second)",
            "sclk_mhz": med, "sclk_mhz_per_xcd": snap[2], "socket_power_w": snap[3],
            "snapshot_after_timed_ms": round((snap[0] - t_end) * 1e3, 1), "extra_launches": n,
            "peak_at_sclk_tflops": round(peak_at, 1), "pct_of_peak_at_sclk": round(100.0 * tflops / peak_at, 2)}


def percentile(xs, q):
    xs = sorted(xs)
    i = min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))
    return xs[i]


class Case:
    """Device-resident inputs (rotated copies) for one workload."""

    def __init__(self, w, torch, gb, rotate=None):
        import numpy as np

        import synth

        self.w = w
        self.torch = torch
        self.gb = gb
        dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32,
              "e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2, "i8": torch.int8, "i32": torch.int32}
        a_bits, b_bits = synth.make_workload(w)
        if w.b_layout:
            b_bits = np.ascontiguousarray(b_bits.T)  # B stored K x N
        raw = np.uint8 if a_bits.dtype == np.uint8 else np.int16
        a = torch.from_numpy(a_bits.view(raw)).to("cuda").view(dt[w.in_dtype])
        b = torch.from_numpy(b_bits.view(raw)).to("cuda").view(dt[w.in_dtype])
        set_bytes = w.compulsory_bytes
        if rotate is None:
            rotate = max(1, -(-2 * MALL_BYTES // set_bytes))  # total touched > 2x the MALL
            rotate = min(rotate, 16)
        self.rotate = rotate
        self.sets = []
        for r in range(rotate):
            ar = a if r == 0 else a.clone()
            br = b if r == 0 else b.clone()
            c = torch.empty(((w.batch,) if w.batch > 1 else ()) + (w.M, w.N), dtype=dt[w.out_dtype], device="cuda")
            self.sets.append((ar, br, c))
        self.in_code = {"bf16": gb.BF16, "f16": gb.F16, "e4m3": gb.FP8_E4M3, "e5m2": gb.FP8_E5M2,
                        "i8": gb.INT8}[w.in_dtype]
        self.out_code = {"f32": gb.F32, "bf16": gb.BF16, "f16": gb.F16, "i32": gb.INT32}[w.out_dtype]
        self.ptrs = [(x.data_ptr(), y.data_ptr(), z.data_ptr()) for x, y, z in self.sets]
        # a single product goes through gemm_bt_ws (the entry point of mm_bt), which splits K where the plan
        # says so; its workspace is allocated and zeroed here, outside the timed region
        self.ws_bytes = 0
        if not w.b_layout and w.batch == 1:
            self.ws_bytes = gb.gemm_bt_workspace_size(w.M, w.N, w.K, self.in_code, self.out_code)
        self.ws = torch.zeros(max(self.ws_bytes, 1), dtype=torch.uint8, device="cuda")
        if not w.b_layout and w.batch == 1:
            self.plan = gb.gemm_bt_plan_ws(w.M, w.N, w.K, self.in_code, self.out_code).as_dict()
        elif w.b_layout:
            self.plan = gb.gemm_bt_plan_layout(w.M, w.N, w.K, gb.K_INNER, w.b_layout, self.in_code,
                                               self.out_code).as_dict()
        else:
            self.plan = gb.gemm_bt_plan_batched(w.batch, w.M, w.N, w.K, self.in_code, self.out_code).as_dict()
        torch.cuda.synchronize()

    def step(self, i, stream):
        pa, pb, pc = self.ptrs[i % self.rotate]
        w = self.w
        if w.b_layout:
            st = self.gb.gemm_bt_layout(pa, pb, pc, w.M, w.N, w.K, self.gb.K_INNER, w.b_layout, self.in_code,
                                        self.out_code, stream)
        elif w.batch > 1:
            st = self.gb.gemm_bt_batched(pa, pb, pc, w.batch, w.M, w.N, w.K, w.M * w.K, w.N * w.K, w.M * w.N,
                                         self.in_code, self.out_code, stream)
        elif self.ws_bytes:
            st = self.gb.gemm_bt_ws(pa, pb, pc, w.M, w.N, w.K, self.in_code, self.out_code, self.ws.data_ptr(),
                                    self.ws_bytes, stream)
        else:
            st = self.gb.gemm_bt(pa, pb, pc, w.M, w.N, w.K, self.in_code, self.out_code, stream)
        if st != self.gb.OK:
            raise self.gb.GemmBtError(st)

    def settle(self, stream, batch=25, min_ms=60.0, max_s=0.6, max_launches=6000, patience=3):
        """Untimed launches until the per-launch time stops falling: batches of `batch` launches for at least
        `min_ms` of load (from idle the 4096^3 launches take 124 us in the second batch and reach their steady
        95-96 us only after 40-55 ms; 1024x4096x4096 first slows from 41 to 48 us, then settles near 39.5 us
        after 30-40 ms), then until `patience` batches in a row are no more than 0.5 % faster than the best so
        far, or at the bounds.  Returns (launches, ms)."""
        torch = self.torch
        sh = stream.cuda_stream
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        best, stale, n = float("inf"), 0, 0
        while True:
            e0.record(stream)
            for i in range(batch):
                self.step(n + i, sh)
            e1.record(stream)
            e1.synchronize()
            n += batch
            per = e0.elapsed_time(e1) / batch
            if per < best * 0.995:
                best, stale = per, 0
            else:
                stale += 1
            elapsed = time.perf_counter() - t0
            if (stale >= patience and elapsed * 1e3 >= min_ms) or elapsed > max_s or n >= max_launches:
                break
        return n, (time.perf_counter() - t0) * 1e3

    def time(self, steps, warmup, settle=True):
        """`warmup` untimed steps, the settle phase, then the `steps` timed steps, back to back between two
        synchronisations (the host wall time of `value`).  Then the same number of launches again behind one
        untimed lead launch, between two HIP events on the launch stream (torch's current stream): their mean
        is the average launch duration.  (Started on an idle stream, the first event would be stamped while
        the host is still issuing the first launch, and that gap, tens of us, would be averaged over the
        launches.)  Then the same number of launches once more, each followed by an event of its own, for the
        spread: an event between two launches also holds the second back by the dispatch gap, so those
        intervals run longer than the launches themselves (by about 1-6 us on MI355X).  Returns a dict: wall
        seconds of the timed steps, event ms of the second pass, the per-launch intervals of the third, the
        settle phase, and the host-clock window of the timed steps."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        sh = stream.cuda_stream
        for i in range(warmup):
            self.step(i, sh)
        torch.cuda.synchronize()
        settle_n, settle_ms = self.settle(stream) if settle else (0, 0.0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(i, sh)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        self.step(steps, sh)  # the lead launch: the stream is busy when e0 is stamped
        e0.record(stream)
        for i in range(steps):
            self.step(i, sh)
        e1.record(stream)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for i in range(steps):
            self.step(i, sh)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
        return {"wall_s": t1 - t0, "event_ms": e0.elapsed_time(e1), "per_ms": per, "settle_launches": settle_n,
                "settle_ms": settle_ms, "t0": t0, "t1": t1}


def timing_record(r):
    per_us = [x * 1e3 for x in r["per_ms"]]
    n = len(per_us)
    return {"launches": n, "mean_us": round(r["event_ms"] * 1e3 / n, 3),
            "per_launch_events": {"median_us": round(percentile(per_us, 0.5), 3), "min_us": round(min(per_us), 3),
                                  "max_us": round(max(per_us), 3), "p10_us": round(percentile(per_us, 0.1), 3),
                                  "p90_us": round(percentile(per_us, 0.9), 3)},
            "settle_launches": r["settle_launches"], "settle_ms": round(r["settle_ms"], 1)}


def cpu_info():
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cpus": affinity}


def cpu_baseline(w, target_s=12.0):
    """The oracle, as it stands, on the first r rows of the product (r sized
    for about `target_s` seconds of host time); value in TFLOP/s."""
    import numpy as np

    import oracle
    import synth

    a_bits, b_bits = synth.make_workload(w)
    threads = oracle.max_threads()
    r = 4
    t0 = time.perf_counter()
    oracle.gemm_bt_ref(a_bits[:r], b_bits, w.in_dtype)
    dt = time.perf_counter() - t0
    rows = int(min(w.M, max(r, r * target_s / max(dt, 1e-6))))
    t0 = time.perf_counter()
    oracle.gemm_bt_ref(a_bits[:rows], b_bits, w.in_dtype)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * w.N * w.K
    rec = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": "rows 0..%d of the %dx%dx%d %s product (%.3g multiply-adds, fp64 triple loop, %d OpenMP "
                     "threads), %.2f s" % (rows - 1, w.M, w.N, w.K, w.in_dtype, rows * w.N * w.K, threads, dt)}
    rec.update(cpu_info())
    return rec


def copy_rate(torch, n=1 << 30, reps=10):
    """GB/s (read + write) of a plain 1 GiB device-to-device copy: the achievable-HBM context."""
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n / ms / 1e6


def copy_mode(torch, steps, warmup):
    """Plain device-to-device copy of 1 GiB, for scaling the HBM byte counters."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    print(json.dumps({"mode": "copy", "bytes_read": n, "bytes_written": n, "ms": ms,
                      "GB/s": 2 * n / ms / 1e6}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--workload", default="sq4096_bf16_bf16")
    ap.add_argument("--rotate", type=int, default=None)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--mode", choices=["gemm", "copy"], default="gemm")
    ap.add_argument("--no-settle", action="store_true",
                    help="skip the settle phase and the clock reading (for counter-collection runs, where the "
                         "profiler serializes every dispatch)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        log("bench.py runs on exactly one GPU: the library is a single-GPU kernel library "
            "(no collectives); --gpus %d is not supported." % args.gpus)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    if args.mode == "copy":
        copy_mode(torch, args.steps, args.warmup)
        return

    import dense_tiled_gemm_amd as gb
    import synth

    gb.load()
    w = synth.WORKLOADS[args.workload]
    log("workload", w)
    case = Case(w, torch, gb, args.rotate)
    plan = case.plan
    log("plan", plan, "rotate", case.rotate, "device CUs", torch.cuda.get_device_properties(0).multi_processor_count)
    sampler = ClockSampler().start()
    r = case.time(args.steps, args.warmup, settle=not args.no_settle)
    ms_per_step = r["wall_s"] / args.steps * 1e3
    tflops = w.flops / (ms_per_step * 1e-3) / 1e12
    timing = timing_record(r)
    achieved = w.flops / (timing["mean_us"] * 1e-6) / 1e12
    clock = clock_under_load(case, sampler, r["t1"], achieved) if not args.no_settle else None
    sampler.stop()
    pl = timing["per_launch_events"]
    log("wall ms/step %.4f  mean launch %.3f us  per-launch events median %.3f (min %.3f, p90 %.3f)  TFLOP/s %.1f "
        "(mean launch %.1f)  settle %d launches / %.1f ms  clock %s" % (
            ms_per_step, timing["mean_us"], pl["median_us"], pl["min_us"], pl["p90_us"], tflops, achieved,
            timing["settle_launches"], timing["settle_ms"], clock))
    traffic = load_traffic(w.name)
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.in_dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "in_dtype": w.in_dtype,
                   "out_dtype": w.out_dtype, "dist": w.dist, "seed": w.seed, "rotated_input_sets": case.rotate,
                   "tile": [plan["bm"], plan["bn"], plan["bk"]], "threads": plan["threads"],
                   "grid": plan["grid"], "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "timing": timing,
        "clock": clock,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
    }
    if not args.no_secondary:
        sec = {}
        for name in ("m1024_n4096_k4096_f16_f16", "skinny_m16_n8192_k8192_bf16_bf16", "sq512_bf16_f32",
                     "ragged_m1000_n3000_k2050_bf16_f32", "sq4096_e4m3_bf16", "sq4096_i8_i32",
                     "batch64_sq512_bf16_bf16", "sq4096_nn_bf16_bf16", "splitk_m1024_n1024_k16384_bf16_bf16",
                     "oddk_m1000_n3000_k2049_bf16_f32", "thin_m64_n8192_k8192_bf16_bf16"):
            w2 = synth.WORKLOADS[name]
            c2 = Case(w2, torch, gb)
            r2 = c2.time(max(50, args.steps // 2) if not args.no_settle else args.steps, args.warmup,
                         settle=not args.no_settle)
            t2 = timing_record(r2)
            us = t2["mean_us"]
            ent = {"us": us, "per_launch_events": t2["per_launch_events"], "launches": t2["launches"],
                   "settle_launches": t2["settle_launches"],
                   "TFLOP/s": round(w2.flops / (us * 1e-6) / 1e12, 2),
                   "GB/s": round(w2.compulsory_bytes / (us * 1e-6) / 1e9, 1),
                   "rotated_input_sets": c2.rotate, "tile": [c2.plan["bm"], c2.plan["bn"], c2.plan["bk"]],
                   "grid": c2.plan["grid"]}
            if c2.plan.get("split_tiles"):
                ent["split_tiles"] = c2.plan["split_tiles"]
            if name.startswith(("skinny", "thin")):  # bound by reading B once
                ent["frac_hbm"] = round(ent["GB/s"] / PEAK_HBM_GBS, 4)
            elif w2.in_dtype in ("e4m3", "e5m2"):
                ent["frac_mfma_fp8"] = round(ent["TFLOP/s"] / PEAK_FP8_TFLOPS, 4)
            elif w2.in_dtype == "i8":  # integer operations: TOP/s
                ent["TOP/s"] = ent.pop("TFLOP/s")
                ent["frac_mfma_i8"] = round(ent["TOP/s"] / PEAK_I8_TOPS, 4)
            else:
                ent["frac_mfma"] = round(ent["TFLOP/s"] / PEAK_BF16_TFLOPS, 4)
            sec[name] = ent
            log(name, ent)
            del c2
            torch.cuda.empty_cache()
        out["secondary"] = sec
        out["copy_GBps"] = round(copy_rate(torch), 1)
        log("copy GB/s", out["copy_GBps"])
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w)
        log("cpu_baseline", out["cpu_baseline"])
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
