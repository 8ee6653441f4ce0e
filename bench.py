#!/usr/bin/env python3
"""Benchmark of C = A·Bᵀ on one MI355X through the libgemm_bt C-ABI.

One step = one gemm_bt call on the 4096×4096×4096 bf16 workload (A and B
i.i.d. N(0,1) rounded to bf16, seed 2, bf16 output), inputs resident in HBM.
Prints ONE JSON line on stdout:
  value        TFLOP/s of the whole job (2·M·N·K per step / step time)
  roofline     the tiled MFMA kernel against the MI355X dense bf16 peak
  cpu_baseline the CPU oracle timed on a bounded sample of the same product
  secondary    µs / TFLOP/s / GB/s of the other workloads (1024×4096×4096
               f16, 16×8192×8192 skinny, 512³, 1000×3000×2050, 4096³ with
               E4M3 inputs against the fp8 peak, 4096³ int8 -> int32
               against the int8 peak, a batch of 64 products of 512³ in one
               gemm_bt_batched call, and 4096³ with B stored K×N through
               gemm_bt_layout), same timing
  copy_GBps    a plain 1 GiB device copy, as context for achievable HBM
Diagnostics go to stderr.  The default 400 untimed warm-up launches matter:
from idle, an MI355X needs about 25 ms of sustained GEMM launches before its
clocks settle, and launches inside that ramp run up to 15% slower.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-secondary]
  python bench.py --mode copy     # plain device copy of known size (counter calibration)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
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
        else:
            st = self.gb.gemm_bt(pa, pb, pc, w.M, w.N, w.K, self.in_code, self.out_code, stream)
        if st != self.gb.OK:
            raise self.gb.GemmBtError(st)

    def time(self, steps, warmup):
        """Returns (wall seconds for `steps` calls, event-measured ms per call)."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        sh = stream.cuda_stream
        for i in range(warmup):
            self.step(i, sh)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(steps):
            self.step(i, sh)
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return t1 - t0, e0.elapsed_time(e1) / steps


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
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "rows 0..%d of the %dx%dx%d %s product (%.3g multiply-adds, fp64 triple loop, %d OpenMP "
                      "threads), %.2f s" % (rows - 1, w.M, w.N, w.K, w.in_dtype, rows * w.N * w.K, threads, dt)}


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
    plan = gb.gemm_bt_plan(w.M, w.N, w.K, case.in_code, case.out_code).as_dict()
    log("plan", plan, "rotate", case.rotate)
    wall, ev_ms = case.time(args.steps, args.warmup)
    ms_per_step = wall / args.steps * 1e3
    tflops = w.flops / (ms_per_step * 1e-3) / 1e12
    achieved = w.flops / (ev_ms * 1e-3) / 1e12
    log("wall ms/step %.4f  event ms/launch %.4f  TFLOP/s %.1f (event %.1f)" % (ms_per_step, ev_ms, tflops,
                                                                                achieved))
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
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
    }
    if not args.no_secondary:
        sec = {}
        for name in ("m1024_n4096_k4096_f16_f16", "skinny_m16_n8192_k8192_bf16_bf16", "sq512_bf16_f32",
                     "ragged_m1000_n3000_k2050_bf16_f32", "sq4096_e4m3_bf16", "sq4096_i8_i32",
                     "batch64_sq512_bf16_bf16", "sq4096_nn_bf16_bf16"):
            w2 = synth.WORKLOADS[name]
            c2 = Case(w2, torch, gb)
            _, ms2 = c2.time(max(50, args.steps // 2), args.warmup)
            ent = {"us": round(ms2 * 1e3, 3), "TFLOP/s": round(w2.flops / (ms2 * 1e-3) / 1e12, 2),
                   "GB/s": round(w2.compulsory_bytes / (ms2 * 1e-3) / 1e9, 1),
                   "rotated_input_sets": c2.rotate}
            if name.startswith("skinny"):
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
