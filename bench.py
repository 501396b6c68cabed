#!/usr/bin/env python3
"""Benchmark: the layout-algebra tiled GEMM on one MI355X.

One step is one D = alpha*A*B + beta*C through the C-ABI library on the
headline workload: bf16 M=N=K=8192, A row-major (K-major), B column-major
(K-major), N(0,1)/sqrt(K) entries, alpha=1, beta=0, fp32 accumulation, bf16
out. Inputs are resident in HBM before the timed region. Prints ONE JSON line
on stdout (everything else goes to stderr):

  value      whole-job TFLOP/s = 2MNK / (wall time per step)
  roofline   the tiled kernel's achieved TFLOP/s from HIP events on the launch
             stream, against the dense bf16 MFMA peak
  cpu_baseline  the fp64 oracle, timed on a bounded sample of the same workload
  extra      the other measured workloads (4096^3 fp16, 6144x4096x2048 M-/N-major
             fp16, and the HBM-bound 32x8192x8192 bf16 in GB/s)

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--only-headline]
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

METRIC = "GEMM TFLOP/s and % of MI355X dense fp16/bf16 MFMA peak at 8192^3 (1 GPU)"
# Dense fp16/bf16 MFMA peak: 256 CUs x 4096 flop/clk/CU x 2.4 GHz = 2516.6
# TFLOP/s (the published 2.5 PFLOP/s, taken at the unit-count value).
PEAK_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("gemm_kernels.hip", "gemm_tiled.hip", "gemm_kernels.hpp", "kernel_common.hpp",
              "device_layout.hpp", "gemm.cpp"):
        h.update(open(os.path.join(ROOT, "layout_algebra_tiled_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_for(kernel_key: str):
    """HBM bytes per launch measured with rocprofv3 counters, if they were
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path)).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


class Workload:
    def __init__(self, cfg: int, n_b: int = 1):
        import torch
        import datagen
        from layout_algebra_tiled_amd.layout import Layout
        self.c = datagen.config(cfg)
        c = self.c
        log(f"[bench] preparing workload {cfg}: {c.name}")
        A, B, C, D = c.make()
        self.host = (A, B, C, D)
        dev = torch.device("cuda:0")
        self.A, self.D = A.to(dev), D.to(dev)
        self.C = C.to(dev) if c.beta != 0 else None
        b0 = B.to(dev)
        # distinct B buffers (same values) so a rotating run streams B from HBM
        # rather than from the 256 MB last-level cache
        self.Bs = [b0] + [datagen.Matrix(b0.store.clone(), b0.shape, b0.stride) for _ in range(n_b - 1)]
        self.lay = {"A": Layout.make(list(A.shape), list(A.stride)), "B": Layout.make(list(B.shape), list(B.stride)),
                    "D": Layout.make(list(D.shape), list(D.stride))}
        if self.C is not None:
            self.lay["C"] = Layout.make(list(C.shape), list(C.stride))

    def plan(self):
        from layout_algebra_tiled_amd import gemm as g
        return g.plan(self.A.store, self.Bs[0].store, self.D.store, self.C.store if self.C is not None else None,
                      self.c.beta, layouts=self.lay)

    def run(self, i: int = 0, workspace=None):
        from layout_algebra_tiled_amd import gemm as g
        g.gemm(self.A.store, self.Bs[i % len(self.Bs)].store, self.D.store,
               self.C.store if self.C is not None else None, self.c.alpha, self.c.beta, layouts=self.lay,
               workspace=workspace)

    def time(self, steps: int, warmup: int, warmup_s: float = 0.0):
        """Wall time per step (barrier + synchronize around the timed steps)
        and the average kernel duration from HIP events on the launch stream.
        Warm-up runs at least `warmup` steps and at least `warmup_s` seconds:
        under sustained MFMA load the GPU's clocks settle only after some
        tens of milliseconds, and the timed steps should see steady state."""
        import torch
        t_end = time.perf_counter() + warmup_s
        i = 0
        while i < warmup or time.perf_counter() < t_end:
            self.run(i)
            i += 1
            if i % 16 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            ev[i][0].record()
            self.run(i)
            ev[i][1].record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        self.kernel_times = sorted(a.elapsed_time(b) / 1e3 for a, b in ev)
        kern = sum(self.kernel_times) / steps
        return wall, kern

    def check(self, npts: int = 256):
        """Sampled parity of the last output against the oracle."""
        import numpy as np
        from oracle import gemm as og
        from tests.gemm_cases import op, sample_points
        import datagen
        A, B, C, _ = self.host
        M, N = self.c.M, self.c.N
        pts = sample_points(M, N, npts, seed=self.c.cfg)
        S, T = og.gemm_points(op(A), op(B), pts)
        Dref, Cabs = og.epilogue(S, op(C) if self.C is not None else None, pts, self.c.alpha, self.c.beta)
        out = datagen.Matrix(self.D.store.cpu(), self.D.shape, self.D.stride)
        return og.check(og.read_points(op(out), pts), Dref, T, Cabs, self.c.alpha, self.c.dtype)


def cpu_baseline(w: Workload, budget_s: float):
    """The oracle as it stands, on a bounded sample: whole output rows of the
    same workload (full K). The oracle spreads rows over its threads, so rows
    go in chunks of one row per thread until about budget_s seconds have run."""
    from oracle import gemm as og
    from tests.gemm_cases import op
    A, B, _, _ = w.host
    Aw, Bw = op(A).widened(), op(B).widened()
    threads = og.num_threads()
    rows, dt = 0, 0.0
    while dt < budget_s and rows < w.c.M:
        chunk = min(threads, w.c.M - rows)
        t0 = time.perf_counter()
        og.gemm_rows(op(A), op(B), range(rows, rows + chunk), Aw=Aw, Bw=Bw)
        dt += time.perf_counter() - t0
        rows += chunk
    flops = 2.0 * rows * w.c.N * w.c.K
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of {w.c.M} output rows of the {w.c.M}x{w.c.N}x{w.c.K} workload, full K "
                      f"({rows * w.c.N} outputs, {dt:.1f} s, fp64 sequential-k sums)"}


def roofline(w: Workload, plan: dict, kern_s: float, traffic):
    """The dominant kernel against its bound: MFMA peak for the tiled and
    16x16 kernels (2MNK flop per launch), HBM peak for the skinny kernel
    (algorithmic bytes per launch: A, B and D once, C once if read)."""
    if plan["kernel_name"] == "skinny":
        gbs = w.c.bytes() / kern_s / 1e9
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic}
    tf = w.c.flops() / kern_s / 1e12
    return {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / PEAK_TFLOPS, 4), "traffic": traffic}


def copy_probe(nbytes: int = 1 << 30, reps: int = 5):
    """A plain device copy of known size through the library's layout gather
    with the identity layout (n):(1): it reads and writes exactly nbytes per
    launch, which calibrates the HBM byte counters against algorithmic bytes."""
    import torch
    from layout_algebra_tiled_amd import gemm as g
    from layout_algebra_tiled_amd.layout import Layout
    n = nbytes // 4
    src = torch.arange(n, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    ident = Layout.make([n], [1])
    g.gather_device(ident, src, dst)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        g.gather_device(ident, src, dst)
        b.record()
    torch.cuda.synchronize()
    if not torch.equal(src, dst):
        raise SystemExit("copy probe: destination differs from source")
    t = sum(a.elapsed_time(b) for a, b in ev) / reps / 1e3
    print(json.dumps({"copy_probe_bytes_read": nbytes, "copy_probe_bytes_written": nbytes, "launches": reps + 1,
                      "us": round(t * 1e6, 1), "GB/s": round(2 * nbytes / t / 1e9, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-headline", action="store_true", help="skip the other workloads (profiling runs)")
    ap.add_argument("--workload", type=int, default=3, help="headline workload (default: bf16 8192^3)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--warmup-seconds", type=float, default=2.0,
                    help="warm up for at least this long as well as --warmup steps (clocks settle)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 1 GiB identity-layout copy (HBM byte-counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the GEMM would shard by N or M with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    from layout_algebra_tiled_amd import gemm as g
    arch = g.device_check()
    log(f"[bench] device {torch.cuda.get_device_name(0)} ({arch})")

    if args.copy_probe:
        copy_probe()
        return

    # the skinny workload's B (128 MiB) would sit in the 256 MB last-level
    # cache between steps: rotate four copies so every step streams B from HBM
    w = Workload(args.workload, n_b=4 if args.workload == 5 else 1)
    plan = w.plan()
    log(f"[bench] plan: {plan['kernel_name']} tile {plan['tile_m']}x{plan['tile_n']}x{plan['tile_k']}, "
        f"wave tile {plan['wave_m']}x{plan['wave_n']}, {plan['waves']} waves, {plan['stages']} LDS stages "
        f"({plan['lds_bytes']} B), grid {plan['grid']}, {plan['mfma_per_wave_kstep']} "
        f"MFMA {plan['mfma_m']}x{plan['mfma_n']}x{plan['mfma_k']} per wave per K step")
    wall, kern = w.time(args.steps, args.warmup, args.warmup_seconds)
    flops = w.c.flops()
    value = flops / wall / 1e12
    achieved = flops / kern / 1e12
    chk = w.check()
    log(f"[bench] {value:.1f} TFLOP/s wall, kernel {kern * 1e6:.1f} us = {achieved:.1f} TFLOP/s; check: {chk}")
    if not chk.ok:
        raise SystemExit(f"bench result failed the oracle check: {chk}")
    tkey = f"{plan['kernel_name']}:workload{args.workload}"
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {torch.bfloat16: "bf16", torch.float16: "f16"}[w.c.dtype],
        "data": "synthetic",
        "config": {"workload": f"{w.c.name}: D = alpha*A*B + beta*C, alpha={w.c.alpha}, beta={w.c.beta}, "
                               f"fp32 accumulate", "M": w.c.M, "N": w.c.N, "K": w.c.K,
                   "kernel": plan["kernel_name"], "tile": [plan["tile_m"], plan["tile_n"], plan["tile_k"]],
                   "grid": plan["grid"], "pct_of_peak": round(100 * value / PEAK_TFLOPS, 2),
                   "kernel_us": {"mean": round(kern * 1e6, 1),
                                 "median": round(w.kernel_times[len(w.kernel_times) // 2] * 1e6, 1),
                                 "min": round(w.kernel_times[0] * 1e6, 1)},
                   "warmup_s": args.warmup_seconds,
                   "parity": f"{chk.n - chk.n_bad}/{chk.n} sampled outputs in bound, worst "
                             f"{chk.worst_fraction:.3f} of budget"},
        "roofline": roofline(w, plan, kern, traffic_for(tkey)),
    }
    if not args.only_headline:
        extra = {}
        for cfg, n_b in ((2, 1), (4, 1), (5, 4)):
            x = Workload(cfg, n_b=n_b)
            p = x.plan()
            ws = None
            if p["workspace_bytes"]:
                ws = torch.empty(p["workspace_bytes"], dtype=torch.uint8, device="cuda:0")
            x.run(0, ws)
            xw, xk = x.time(max(10, args.steps // 2), 5, args.warmup_seconds / 2)
            xc = x.check(128)
            rec = {"kernel": p["kernel_name"], "ms_per_step": round(xw * 1e3, 4), "kernel_us": round(xk * 1e6, 2),
                   "TFLOP/s": round(x.c.flops() / xw / 1e12, 2), "parity_ok": bool(xc.ok),
                   "worst_fraction": round(xc.worst_fraction, 4)}
            if cfg == 5:
                rec["GB/s"] = round(x.c.bytes() / xk / 1e9, 1)
                rec["frac_hbm"] = round(x.c.bytes() / xk / 1e9 / PEAK_HBM_GBS, 4)
                rec["B_buffers_rotated"] = n_b
            else:
                rec["pct_of_peak"] = round(100 * x.c.flops() / xk / 1e12 / PEAK_TFLOPS, 2)
            extra[f"workload{cfg}: {x.c.name}"] = rec
            log(f"[bench] workload {cfg}: {rec}")
            del x
            torch.cuda.empty_cache()
        line["extra"] = extra
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
        log(f"[bench] cpu baseline: {line['cpu_baseline']}")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
