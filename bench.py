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
  extra      the other measured workloads (256x128x64 fp16, 4096^3 fp16,
             6144x4096x2048 M-/N-major fp16, the HBM-bound 32x8192x8192 bf16 in
             GB/s), a shape whose tiles leave CUs idle with and without the split
             remainder, and the device layout map
The sampled checks here are fp64 torch sums on the device; the oracle runs
only in the CPU-baseline leg (its parity claims live in tests/).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--only-headline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
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
              "device_layout.hpp", "tiled_config.hpp", "gemm.cpp"):
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


class GpuSensors:
    """Shader clock and board power of cuda:0 from the driver's sysfs files of
    its PCI device (plain file reads: no other program is started). Each read
    returns None where the files are absent or unreadable."""

    def __init__(self):
        import glob
        import torch
        self.sclk_path = self.power_path = None
        try:
            pr = torch.cuda.get_device_properties(0)
            dev = f"/sys/bus/pci/devices/{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}.0"
        except Exception:
            return
        hw = sorted(glob.glob(dev + "/hwmon/hwmon*/"))
        for name, attr in (("freq1_input", "sclk_path"), ("power1_input", "power_path")):
            for d in hw:
                if os.access(d + name, os.R_OK):
                    setattr(self, attr, d + name)
                    break
        if self.sclk_path is None and os.access(dev + "/pp_dpm_sclk", os.R_OK):
            self.sclk_path = dev + "/pp_dpm_sclk"

    @staticmethod
    def _read(path):
        try:
            return open(path).read() if path else None
        except OSError:
            return None

    def sclk_mhz(self):
        text = self._read(self.sclk_path)
        if text is None:
            return None
        try:
            if self.sclk_path.endswith("freq1_input"):
                return int(text.split()[0]) / 1e6
            for line in text.splitlines():   # the current level ends with '*': "S: 1803Mhz *"
                if line.rstrip().endswith("*"):
                    return float(line.split(":")[1].split()[0].lower().replace("mhz", ""))
        except (ValueError, IndexError):
            return None
        return None

    def power_w(self):
        text = self._read(self.power_path)
        try:
            return int(text.split()[0]) / 1e6 if text else None
        except (ValueError, IndexError):
            return None


class StreamHold:
    """Holds the current stream for a while with a bounded spin kernel
    (torch.cuda._sleep), so that the launches queued behind it run back to
    back: HIP events around each launch then time the kernel, not the host's
    marshalling between launches (which exceeds a short kernel's duration)."""

    def __init__(self):
        import torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 1 << 22
        torch.cuda._sleep(n // 16)   # first launch outside the calibration
        torch.cuda.synchronize()
        e0.record()
        torch.cuda._sleep(n)
        e1.record()
        torch.cuda.synchronize()
        self.cycles_per_ms = n / max(e0.elapsed_time(e1), 1e-3)

    def hold(self, ms: float):
        import torch
        torch.cuda._sleep(int(self.cycles_per_ms * ms))


_HOLD = None


def queued_kernel_times(run, n: int):
    """Per-launch kernel durations (s) of n launches run(i) queued behind a
    stream hold long enough for the host to enqueue all of them."""
    import torch
    global _HOLD
    if _HOLD is None:
        _HOLD = StreamHold()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    _HOLD.hold(2.0 + 0.2 * n)
    for i in range(n):
        ev[i][0].record()
        run(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) / 1e3 for a, b in ev)


def queued_block_time(run, n: int):
    """Mean duration (s) of n launches run(i) queued back to back behind a
    stream hold, from one pair of HIP events around all of them: no event
    between launches, so short kernels are not charged the event overhead
    (about 2 us per launch here) that per-launch events add."""
    import torch
    global _HOLD
    if _HOLD is None:
        _HOLD = StreamHold()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    _HOLD.hold(2.0 + 0.2 * n)
    e0.record()
    for i in range(n):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / n


class Workload:
    def __init__(self, cfg: int, n_b: int = 1, mnk=None, beta=None, persistent=None):
        import dataclasses
        import torch
        import datagen
        from layout_algebra_tiled_amd.layout import Layout
        self.c = datagen.config(cfg)
        if mnk:
            self.c = dataclasses.replace(self.c, M=mnk[0], N=mnk[1], K=mnk[2],
                                         name=f"{self.c.name} at {mnk[0]}x{mnk[1]}x{mnk[2]}")
        if beta is not None:
            self.c = dataclasses.replace(self.c, beta=beta, name=f"{self.c.name} with beta={beta}")
        c = self.c
        self.persistent = persistent   # None: the planner's choice
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
                      self.c.beta, layouts=self.lay, persistent=self.persistent)

    def run(self, i: int = 0):
        from layout_algebra_tiled_amd import gemm as g
        if not hasattr(self, "ws"):
            import torch
            need = self.plan()["workspace_bytes"]
            self.ws = torch.empty(need, dtype=torch.uint8, device="cuda:0") if need else None
        g.gemm(self.A.store, self.Bs[i % len(self.Bs)].store, self.D.store,
               self.C.store if self.C is not None else None, self.c.alpha, self.c.beta, layouts=self.lay,
               workspace=self.ws, persistent=self.persistent)

    def queued_kernel_time(self, steps: int):
        """Mean kernel duration (s) of `steps` launches queued back to back
        behind a stream hold (HIP events around each launch)."""
        t = queued_kernel_times(self.run, steps)
        self.queued_times = t
        return sum(t) / len(t)

    def time(self, steps: int, warmup: int, warmup_s: float = 0.0, sample_clock: bool = False):
        """Wall time per step (barrier + synchronize around the timed steps)
        and the average kernel duration from HIP events on the launch stream,
        recorded around each launch inside the timed region.
        Warm-up runs at least `warmup` steps and at least `warmup_s` seconds:
        under sustained MFMA load the GPU's clocks settle only after some
        tens of milliseconds, and the timed steps should see steady state."""
        import torch
        t0 = time.perf_counter()
        t_end = t0 + warmup_s
        i = 0
        sensors = GpuSensors() if sample_clock else None
        sclk, power = [], []
        while i < warmup or time.perf_counter() < t_end:
            self.run(i)
            i += 1
            if i % 16 == 0:
                # sampled while the 16 launches just queued are running
                if sensors is not None and time.perf_counter() - t0 > 0.5 * warmup_s:
                    for lst, v in ((sclk, sensors.sclk_mhz()), (power, sensors.power_w())):
                        if v is not None:
                            lst.append(v)
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        self.sclk_mhz = round(sum(sclk) / len(sclk), 1) if sclk else None
        self.power_w = round(sum(power) / len(power), 1) if power else None
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
        """Sampled sanity check of the last output (fp64 dot products on the
        GPU at corner, edge and random outputs; the oracle parity tests cover
        these launches in tests/)."""
        A, B, C, _ = self.host
        return sample_check(self.A.view(), self.Bs[0].view(), self.C.view() if self.C is not None else None,
                            self.D.view(), self.c.alpha, self.c.beta, self.c.dtype,
                            sample_points(self.c.M, self.c.N, npts, seed=self.c.cfg))


class Check:
    def __init__(self, n, n_bad, worst, nonfinite):
        self.n, self.n_bad, self.worst_fraction, self.nonfinite = n, n_bad, worst, nonfinite
        self.ok = n_bad == 0

    def __str__(self):
        return (f"{self.n - self.n_bad}/{self.n} within bound, worst {self.worst_fraction:.4f} of budget, "
                f"non-finite {self.nonfinite}")


def sample_points(M: int, N: int, n: int, seed: int):
    """Corners, edges and n uniform random outputs."""
    import numpy as np
    rng = np.random.default_rng(seed)
    pts = [(0, 0), (0, N - 1), (M - 1, 0), (M - 1, N - 1)]
    pts += [(i, j) for i in (0, M - 1) for j in range(0, N, max(1, N // 64))]
    pts += [(i, j) for j in (0, N - 1) for i in range(0, M, max(1, M // 64))]
    r = np.stack([rng.integers(0, M, n), rng.integers(0, N, n)], axis=1)
    return np.concatenate([np.array(pts, dtype=np.int64), r.astype(np.int64)])


def sample_check(A, B, C, D, alpha: float, beta: float, dtype, pts) -> Check:
    """|D - D_ref| <= 2e-3 (|alpha| sum_k |a b| + |beta c|) + one output ulp at
    the given outputs, D_ref in fp64 from the same 16-bit inputs (torch on the
    device: A (M,K), B (K,N), C, D (M,N) strided views)."""
    import torch
    i = torch.as_tensor(pts[:, 0], device=A.device)
    j = torch.as_tensor(pts[:, 1], device=A.device)
    prod = A.index_select(0, i).double() * B.index_select(1, j).t().double()
    S, T = prod.sum(1), prod.abs().sum(1)
    ref = alpha * S
    cabs = torch.zeros_like(S)
    if C is not None and beta != 0.0:
        c = C[i, j].double()
        ref = ref + beta * c
        cabs = (beta * c).abs()
    p, emin = {torch.float16: (10, -14), torch.bfloat16: (7, -126)}[dtype]
    e = torch.floor(torch.log2(ref.abs().clamp_min(2.0 ** emin))).clamp_min(emin)
    bound = 2e-3 * (abs(alpha) * T + cabs) + torch.exp2(e - p)
    got = D[i, j].double()
    finite = torch.isfinite(got)
    err = torch.where(finite, (got - ref).abs(), torch.full_like(got, float("inf")))
    frac = err / bound
    bad = ~(err <= bound)
    return Check(len(pts), int(bad.sum()), float(frac.max()) if len(pts) else 0.0, int((~finite).sum()))


def cpu_baseline(w: Workload, budget_s: float):
    """The oracle as it stands, on a bounded sample: whole output rows of the
    same workload (full K). The oracle spreads rows over its threads, so rows
    go in chunks of one row per thread until about budget_s seconds have run."""
    from oracle import gemm as og
    from oracle.gemm import Operand
    op = lambda m: Operand(m.store, m.shape, m.stride)
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
    # the layout oracle beside the device layout map (reported only)
    from oracle import layout as ol
    t0 = time.perf_counter()
    ol.enumerate_offsets(ol.zipped_divide(ol.parse_layout("(256,128):(128,1)"), (16, 16)))
    lay_ms = (time.perf_counter() - t0) * 1e3
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of {w.c.M} output rows of the {w.c.M}x{w.c.N}x{w.c.K} workload, full K "
                      f"({rows * w.c.N} outputs, {dt:.1f} s, fp64 sequential-k sums)",
            "layout_map_oracle_ms": round(lay_ms, 1),
            "layout_map_sample": "enumeration of zipped_divide((256,128):(128,1),(16,16)), 32768 offsets, 1 thread"}


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


def torch_matmul_timing(w: Workload, steps: int):
    """torch.matmul (the vendor GEMM library) on the same operands, for scale:
    queued launches after a warm-up, HIP events around each."""
    import torch
    A, B = w.A.view(), w.Bs[0].view()
    out = torch.empty(w.c.M, w.c.N, dtype=w.c.dtype, device="cuda:0")
    run = lambda i: torch.matmul(A, B, out=out)
    t_end = time.perf_counter() + 1.0
    while time.perf_counter() < t_end:
        for _ in range(8):
            run(0)
        torch.cuda.synchronize()
    ts = queued_kernel_times(run, steps)
    mean = sum(ts) / len(ts)
    return {"us_mean": round(mean * 1e6, 1), "us_min": round(ts[0] * 1e6, 1),
            "TFLOP/s": round(w.c.flops() / mean / 1e12, 1)}


# bf16, K-major A and B, N-major D, alpha = 1, beta = 0 (the headline's
# layouts): squares, then shapes of the kind a transformer's linear layers
# run (hidden 4096 with an 11008 or 14336 MLP width, 8192 with 28672), and a
# short-K and a long-K one
SWEEP_SHAPES = [(n, n, n) for n in (1024, 2048, 3072, 4096, 6144, 8192, 12288, 16384)] + [
    (4096, 11008, 4096), (4096, 4096, 11008), (8192, 14336, 4096), (8192, 28672, 8192), (16384, 16384, 1024),
    (2048, 2048, 32768)]


def sweep(reps: int = 8, launches: int = 10):
    """Ours against torch.matmul (the vendor GEMM library) on the same
    operands over SWEEP_SHAPES: launches queued back to back behind a stream
    hold, one event pair per block, the two libraries alternating block by
    block; the median block of each. Operands are drawn on the device from a
    seeded generator (N(0,1)/sqrt(K), rounded to bf16). One JSON line per
    shape on stdout. Timing only: the parity tests check these kernels."""
    import torch
    from layout_algebra_tiled_amd import gemm as g
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261202)
    for M, N, K in SWEEP_SHAPES:
        A = (torch.randn(M, K, device=dev, generator=gen) / math.sqrt(K)).to(torch.bfloat16)
        Bt = (torch.randn(N, K, device=dev, generator=gen) / math.sqrt(K)).to(torch.bfloat16)
        B = Bt.t()   # K x N, K-major
        D, D2 = (torch.empty(M, N, dtype=torch.bfloat16, device=dev) for _ in range(2))
        plan = g.plan(A, B, D)
        need = plan["workspace_bytes"]
        ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
        runs = {"ours": lambda i: g.gemm(A, B, D, workspace=ws),
                "torch.matmul": lambda i: torch.matmul(A, B, out=D2)}
        t_end = time.perf_counter() + 0.5
        while time.perf_counter() < t_end:
            for r in runs.values():
                r(0)
            torch.cuda.synchronize()
        t = {k: [] for k in runs}
        names = list(runs)
        for rep in range(reps):
            for k in (names if rep % 2 == 0 else names[::-1]):
                t[k].append(queued_block_time(runs[k], launches))
        flops = 2.0 * M * N * K
        rec = {"M": M, "N": N, "K": K, "plan": {k: plan[k] for k in ("kernel_name", "tile_m", "tile_n", "grid",
                                                                     "persistent", "tile_order", "split_k",
                                                                     "sk_tiles")}}
        for k, v in t.items():
            med = sorted(v)[len(v) // 2]
            rec[k] = {"us": round(med * 1e6, 1), "TFLOP/s": round(flops / med / 1e12, 1),
                      "frac": round(flops / med / 1e12 / PEAK_TFLOPS, 4)}
        rec["ours_vs_torch"] = round(rec["torch.matmul"]["us"] / rec["ours"]["us"], 3)
        print(json.dumps(rec), flush=True)
        del A, Bt, B, D, D2, ws
        torch.cuda.empty_cache()


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


def layout_map_timing(reps: int = 20):
    """The layout-map path: the device evaluation of zipped_divide((256,128):
    (128,1), (16,16)) (32,768 offsets) timed with HIP events, compared with
    the host library's evaluation of the same layout (the oracle parity of
    both is in tests/; the oracle's own enumeration time is reported in the
    CPU baseline)."""
    import torch
    from layout_algebra_tiled_amd import gemm as g
    from layout_algebra_tiled_amd.layout import Layout
    L = Layout.parse("(256,128):(128,1)").zipped_divide((16, 16))
    n = L.size()
    out = torch.empty(n, dtype=torch.int64, device="cuda:0")
    g.layout_eval_device(L, out)
    torch.cuda.synchronize()
    ts = queued_kernel_times(lambda i: g.layout_eval_device(L, out), reps)
    dev_s = sum(ts) / reps
    same = out.cpu().tolist() == [L(x) for x in range(n)]
    return {"layout": str(L), "elements": n, "device_us": round(dev_s * 1e6, 2),
            "equals_host_library": bool(same)}


def split_remainder_timing(M: int, N: int, K: int, reps: int = 20):
    """A bf16 shape whose tiles fill no whole round of the 256 CUs, timed with
    the split turned off (split_k=1: the planner then takes whole tiles of
    its choice) and with the planner's choice (the last round's 256x256
    tiles split into K segments), plus a sampled fp64 check of the split
    result."""
    import torch
    import datagen
    from layout_algebra_tiled_amd import gemm as g
    A = datagen.matrix(M, K, torch.bfloat16, "row", "normal_over_sqrtk", 11, ld=K, k_for_scale=K)
    B = datagen.matrix(K, N, torch.bfloat16, "col", "normal_over_sqrtk", 12, ld=K, k_for_scale=K)
    dA, dB = A.to("cuda:0"), B.to("cuda:0")
    D = torch.empty(M, N, dtype=torch.bfloat16, device="cuda:0")
    rec = {"shape": f"bf16 {M}x{N}x{K}, K-major A and B"}
    for label, split in (("whole_tiles", 1), ("planned", 0)):
        p = g.plan(dA.view(), dB.view(), D, None, 0.0, kernel="tiled", split_k=split)
        ws = torch.empty(max(p["workspace_bytes"], 1), dtype=torch.uint8, device="cuda:0")
        run = lambda: g.gemm(dA.view(), dB.view(), D, None, 1.0, 0.0, kernel="tiled", split_k=split, workspace=ws)
        t_end = time.perf_counter() + 0.5
        while time.perf_counter() < t_end:
            run()
            torch.cuda.synchronize()
        ts = queued_kernel_times(lambda i: run(), reps)
        k = sum(ts) / reps
        rec[label] = {"tile": [p["tile_m"], p["tile_n"]], "grid": p["grid"], "split_tiles": p["sk_tiles"],
                      "segments": p["split_k"],
                      "kernel_us": round(k * 1e6, 1), "TFLOP/s": round(2 * M * N * K / k / 1e12, 1)}
    chk = sample_check(dA.view(), dB.view(), None, D, 1.0, 0.0, torch.bfloat16, sample_points(M, N, 500, seed=7))
    rec["parity"] = str(chk)
    rec["parity_ok"] = bool(chk.ok)
    return rec


def persistent_timing(reps: int = 5, n: int = 20):
    """The fp16 6144x4096x2048 M-/N-major workload (alpha = 2, beta = -1;
    the planner takes the persistent launch of its 256x128 tiles) timed both
    ways, interleaved: persistent and one workgroup per tile, each as the
    median over `reps` blocks of n launches queued back to back; plus a
    sampled check of the persistent result."""
    import torch
    ws = {"persistent": Workload(4, persistent=None), "one_per_tile": Workload(4, persistent=False)}
    rec = {"shape": "fp16 6144x4096x2048, M-major A, N-major B, alpha=2, beta=-1 (256x128 tiles)"}
    for w in ws.values():
        w.run(0)
    t_end = time.perf_counter() + 0.5
    while time.perf_counter() < t_end:
        for w in ws.values():
            for i in range(4):
                w.run(i)
        torch.cuda.synchronize()
    res = {k: [] for k in ws}
    for _ in range(reps):
        for k, w in ws.items():
            res[k].append(queued_block_time(w.run, n))
    for k, w in ws.items():
        p = w.plan()
        t = sorted(res[k])[reps // 2]
        rec[k] = {"grid": p["grid"], "persistent": bool(p["persistent"]), "kernel_us_back_to_back": round(t * 1e6, 1),
                  "TFLOP/s": round(w.c.flops() / t / 1e12, 1)}
    ws["persistent"].run(0)
    chk = ws["persistent"].check(256)
    rec["parity"] = str(chk)
    rec["parity_ok"] = bool(chk.ok)
    return rec


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
    ap.add_argument("--mnk", type=str, default=None,
                    help="M,N,K: the headline workload's layouts and distributions at another size (profiling "
                         "runs; the reported metric is defined at 8192^3 only)")
    ap.add_argument("--beta", type=float, default=None,
                    help="the headline workload with another beta (profiling runs)")
    ap.add_argument("--persistent", choices=("auto", "on", "off"), default="auto",
                    help="the persistent launch of 256x128 tiles: the planner's choice, forced on or off "
                         "(profiling runs)")
    ap.add_argument("--sweep", action="store_true",
                    help="only time ours against torch.matmul over a list of bf16 shapes (one JSON line each)")
    ap.add_argument("--also-torch-matmul", action="store_true",
                    help="also time torch.matmul (the vendor GEMM library) on the same operands, for scale")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the GEMM would shard by N or M with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    if not args.no_cpu_baseline:
        # compile the C oracle (if stale) before the GPU is touched: a process
        # that has initialised the GPU must not start other programs
        from oracle import gemm as og
        og.build()
    import torch
    from layout_algebra_tiled_amd import gemm as g
    arch = g.device_check()
    log(f"[bench] device {torch.cuda.get_device_name(0)} ({arch})")

    if args.copy_probe:
        copy_probe()
        return
    if args.sweep:
        sweep()
        return

    # the skinny workload's B (128 MiB) would sit in the 256 MB last-level
    # cache between steps: rotate four copies so every step streams B from HBM
    mnk = tuple(int(x) for x in args.mnk.split(",")) if args.mnk else None
    pers = {"auto": None, "on": True, "off": False}[args.persistent]
    w = Workload(args.workload, n_b=4 if args.workload == 5 else 1, mnk=mnk, beta=args.beta, persistent=pers)
    plan = w.plan()
    log(f"[bench] plan: {plan['kernel_name']} tile {plan['tile_m']}x{plan['tile_n']}x{plan['tile_k']}, "
        f"wave tile {plan['wave_m']}x{plan['wave_n']}, {plan['waves']} waves, {plan['stages']} LDS stages "
        f"({plan['lds_bytes']} B), grid {plan['grid']}, {plan['mfma_per_wave_kstep']} "
        f"MFMA {plan['mfma_m']}x{plan['mfma_n']}x{plan['mfma_k']} per wave per K step")
    wall, kern = w.time(args.steps, args.warmup, args.warmup_seconds, sample_clock=True)
    flops = w.c.flops()
    value = flops / wall / 1e12
    achieved = flops / kern / 1e12
    # after the timed region: the same launches queued back to back between
    # one pair of events (no event between launches)
    b2b = queued_block_time(w.run, args.steps)
    chk = w.check()
    log(f"[bench] {value:.1f} TFLOP/s wall, kernel {kern * 1e6:.1f} us = {achieved:.1f} TFLOP/s "
        f"(back to back {b2b * 1e6:.1f} us); check: {chk}")
    if not chk.ok:
        raise SystemExit(f"bench result failed the sampled check: {chk}")
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
                   "grid": plan["grid"], "persistent": bool(plan["persistent"]),
                   "tile_order": {0: None, 1: "raster", 2: "superblock", 3: "raster_krev"}[plan["tile_order"]],
                   "pct_of_peak": round(100 * value / PEAK_TFLOPS, 2),
                   "kernel_us": {"mean": round(kern * 1e6, 1),
                                 "median": round(w.kernel_times[len(w.kernel_times) // 2] * 1e6, 1),
                                 "min": round(w.kernel_times[0] * 1e6, 1),
                                 "back_to_back": round(b2b * 1e6, 1)},
                   "warmup_s": args.warmup_seconds,
                   "sclk_mhz_under_load": w.sclk_mhz,
                   "board_power_w_under_load": w.power_w,
                   "peak_at_sclk_TFLOPs": (round(256 * 4096 * w.sclk_mhz * 1e6 / 1e12, 1)
                                           if w.sclk_mhz else None),
                   "parity": f"{chk.n - chk.n_bad}/{chk.n} sampled outputs in bound, worst "
                             f"{chk.worst_fraction:.3f} of budget"},
        "roofline": roofline(w, plan, kern, traffic_for(tkey)),
    }
    if args.also_torch_matmul:
        line["torch_matmul"] = torch_matmul_timing(w, args.steps)
        log(f"[bench] torch.matmul on the same operands: {line['torch_matmul']}")
    if not args.only_headline:
        extra = {}
        for cfg, n_b in ((1, 1), (2, 1), (4, 1), (5, 4)):
            x = Workload(cfg, n_b=n_b)
            p = x.plan()
            x.run(0)
            n = max(10, args.steps // 2)
            xw, _ = x.time(n, 5, args.warmup_seconds / 2)
            # launches queued back to back: the kernel's own duration (the
            # small workloads are host-bound at one Python call per step)
            xk = x.queued_kernel_time(n)
            xb = queued_block_time(x.run, n)
            xc = x.check(128)
            rec = {"kernel": p["kernel_name"], "tile": [p["tile_m"], p["tile_n"], p["tile_k"]], "grid": p["grid"],
                   "persistent": bool(p["persistent"]),
                   "ms_per_step": round(xw * 1e3, 4), "kernel_us": round(xk * 1e6, 2),
                   "kernel_us_median": round(x.queued_times[len(x.queued_times) // 2] * 1e6, 2),
                   "kernel_us_back_to_back": round(xb * 1e6, 2),
                   "TFLOP/s": round(x.c.flops() / xk / 1e12, 2), "parity_ok": bool(xc.ok),
                   "worst_fraction": round(xc.worst_fraction, 4)}
            if cfg == 1:
                rec["note"] = "launch-latency bound: 128 16x16 tiles, one wave each"
            if cfg == 5:
                # bytes per launch over the back-to-back duration (the
                # per-launch events add about 2 us to a 25 us kernel)
                rec["GB/s"] = round(x.c.bytes() / xb / 1e9, 1)
                rec["frac_hbm"] = round(x.c.bytes() / xb / 1e9 / PEAK_HBM_GBS, 4)
                rec["GB/s_per_launch_events"] = round(x.c.bytes() / xk / 1e9, 1)
                rec["B_buffers_rotated"] = n_b
            else:
                rec["pct_of_peak"] = round(100 * x.c.flops() / xk / 1e12 / PEAK_TFLOPS, 2)
            extra[f"workload{cfg}: {x.c.name}"] = rec
            log(f"[bench] workload {cfg}: {rec}")
            del x
            torch.cuda.empty_cache()
        extra["split remainder (8192x8448x8192, 1,056 tiles)"] = split_remainder_timing(8192, 8448, 8192, reps=10)
        log(f"[bench] split remainder: {extra['split remainder (8192x8448x8192, 1,056 tiles)']}")
        extra["persistent launch (6144x4096x2048)"] = persistent_timing()
        log(f"[bench] persistent launch: {extra['persistent launch (6144x4096x2048)']}")
        extra["layout map"] = layout_map_timing()
        log(f"[bench] layout map: {extra['layout map']}")
        line["extra"] = extra
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
        log(f"[bench] cpu baseline: {line['cpu_baseline']}")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
