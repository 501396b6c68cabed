"""Shared helpers of the GEMM parity tests and the smoke check: build a seeded
case, run it through the C-ABI library on the GPU, and compare with the
oracle element by element (all outputs, or sampled outputs at full size)."""

from __future__ import annotations

import sys
from typing import Optional

import numpy as np
import torch

import datagen
from oracle import gemm as og


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def op(m: datagen.Matrix) -> og.Operand:
    return og.Operand(m.store, m.shape, m.stride)


def sample_points(M: int, N: int, n: int, seed: int) -> np.ndarray:
    """Corner and edge outputs plus n uniform random ones."""
    rng = np.random.default_rng(seed)
    pts = [(0, 0), (0, N - 1), (M - 1, 0), (M - 1, N - 1)]
    pts += [(i, j) for i in (0, M - 1) for j in range(0, N, max(1, N // 64))]
    pts += [(i, j) for j in (0, N - 1) for i in range(0, M, max(1, M // 64))]
    r = np.stack([rng.integers(0, M, n), rng.integers(0, N, n)], axis=1)
    return np.concatenate([np.array(pts, dtype=np.int64), r.astype(np.int64)])


def all_points(M: int, N: int) -> np.ndarray:
    i, j = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    return np.stack([i.reshape(-1), j.reshape(-1)], axis=1).astype(np.int64)


def run_gemm(A: datagen.Matrix, B: datagen.Matrix, C: Optional[datagen.Matrix], D: datagen.Matrix,
             alpha: float, beta: float, kernel="auto", split_k: int = 0, tile=None,
             expect_kernel: Optional[str] = None, label: str = "", persistent=None, tile_order=None):
    """Run D = alpha*A*B + beta*C on cuda:0 through the library, D pre-filled
    with NaN (an output the kernel never writes fails any check). Returns
    (plan dict, output matrix on the CPU)."""
    from layout_algebra_tiled_amd import gemm as g
    from layout_algebra_tiled_amd.layout import Layout

    M, N = D.shape
    say(f"[gemm] {label} M={M} N={N} K={A.shape[1]} {A.dtype} A{A.stride} B{B.stride} D{D.stride} "
        f"alpha={alpha} beta={beta} kernel={kernel} tile={tile} split_k={split_k} persistent={persistent} "
        f"tile_order={tile_order}")
    dev = torch.device("cuda:0")
    dA, dB, dD = A.to(dev), B.to(dev), D.to(dev)
    dC = C.to(dev) if C is not None else None
    dD.store.fill_(float("nan"))
    lay = {"A": Layout.make(list(A.shape), list(A.stride)), "B": Layout.make(list(B.shape), list(B.stride)),
           "D": Layout.make(list(D.shape), list(D.stride))}
    if C is not None:
        lay["C"] = Layout.make(list(C.shape), list(C.stride))
    plan = g.plan(dA.store, dB.store, dD.store, dC.store if dC is not None else None, beta, kernel=kernel,
                  tile=tile, split_k=split_k, layouts=lay, persistent=persistent, tile_order=tile_order)
    if expect_kernel:
        assert plan["kernel_name"] == expect_kernel, plan
    g.gemm(dA.store, dB.store, dD.store, dC.store if dC is not None else None, alpha, beta, kernel=kernel,
           tile=tile, split_k=split_k, layouts=lay, persistent=persistent, tile_order=tile_order)
    torch.cuda.synchronize()
    out = datagen.Matrix(dD.store.cpu(), D.shape, D.stride)
    say(f"[gemm] {label} ran {plan['kernel_name']} tile {plan['tile_m']}x{plan['tile_n']} grid={plan['grid']} "
        f"split_k={plan['split_k']}")
    return plan, out


def check_points(A, B, C, out, alpha, beta, points) -> og.CheckResult:
    S, T = og.gemm_points(op(A), op(B), points)
    Dref, Cabs = og.epilogue(S, op(C) if C is not None else None, points, alpha, beta)
    got = og.read_points(op(out), points)
    return og.check(got, Dref, T, Cabs, alpha, A.dtype)


def _kmajor(m: datagen.Matrix, k_mode: int) -> og.Operand:
    """The same values with K contiguous (an exact copy in another memory
    order), so the oracle's sequential-k loop walks memory in order."""
    v = m.view()
    if k_mode == 1:   # A (M,K): rows of K
        return og.Operand(v.contiguous().reshape(-1), m.shape, (m.shape[1], 1))
    return og.Operand(v.t().contiguous().reshape(-1), m.shape, (1, m.shape[0]))   # B (K,N): columns of K


def check_all_rows(A, B, C, out, alpha, beta, chunk: int = 512) -> og.CheckResult:
    """Every output checked against the oracle, whole rows at a time (bounded
    memory at any size)."""
    M, N = out.shape
    oa, ob = _kmajor(A, 1), _kmajor(B, 0)
    Aw, Bw = oa.widened(), ob.widened()
    oc, oo = (op(C) if C is not None else None), op(out)
    n = n_bad = nonfinite = 0
    worst, worst_i = 0.0, -1
    for r0 in range(0, M, chunk):
        rows = np.arange(r0, min(M, r0 + chunk), dtype=np.int64)
        S, T = og.gemm_rows(oa, ob, rows, Aw=Aw, Bw=Bw)
        ii, jj = np.meshgrid(rows, np.arange(N, dtype=np.int64), indexing="ij")
        pts = np.stack([ii.reshape(-1), jj.reshape(-1)], axis=1)
        Dref, Cabs = og.epilogue(S.reshape(-1), oc, pts, alpha, beta)
        res = og.check(og.read_points(oo, pts), Dref, T.reshape(-1), Cabs, alpha, A.dtype)
        if res.worst_fraction > worst or worst_i < 0:
            worst, worst_i = res.worst_fraction, n + res.worst_index
        n += res.n
        n_bad += res.n_bad
        nonfinite += res.nonfinite
    return og.CheckResult(ok=n_bad == 0, n=n, n_bad=n_bad, worst_fraction=worst, worst_index=worst_i,
                          nonfinite=nonfinite)


def run_and_check(A: datagen.Matrix, B: datagen.Matrix, C: Optional[datagen.Matrix], D: datagen.Matrix,
                  alpha: float, beta: float, points: Optional[np.ndarray] = None, kernel="auto",
                  split_k: int = 0, tile=None, expect_kernel: Optional[str] = None, label: str = "",
                  persistent=None):
    """Run D = alpha*A*B + beta*C on cuda:0 through the library and check the
    result against the oracle (every output, or the given points). Returns
    (CheckResult, plan dict, output)."""
    M, N = D.shape
    plan, out = run_gemm(A, B, C, D, alpha, beta, kernel=kernel, split_k=split_k, tile=tile,
                         expect_kernel=expect_kernel, label=label, persistent=persistent)
    res = check_points(A, B, C, out, alpha, beta, all_points(M, N) if points is None else points)
    say(f"[gemm] {label} {plan['kernel_name']} grid={plan['grid']} split_k={plan['split_k']}: {res}")
    return res, plan, out


def run_and_check_fused(A: datagen.Matrix, B: datagen.Matrix, C: Optional[datagen.Matrix], D: datagen.Matrix,
                        alpha: float, beta: float, bias: Optional[torch.Tensor], bias_per_row: bool,
                        act: Optional[str], kernel="auto", split_k: int = 0, bias_stride: int = 1,
                        expect_kernel: Optional[str] = None, label: str = "", tile=None, persistent=None):
    """The fused epilogue D = act(alpha*A*B + beta*C + bias) through
    lt_gemm_run_ex, every output checked against the oracle; also returns the
    kernel's max |D| and the max over the output it wrote."""
    from layout_algebra_tiled_amd import gemm as g
    from layout_algebra_tiled_amd.layout import Layout

    M, N = D.shape
    say(f"[gemm-fused] {label} M={M} N={N} K={A.shape[1]} {A.dtype} bias={'row' if bias_per_row else 'col'}"
        f"{'' if bias is not None else '(none)'} act={act} kernel={kernel} split_k={split_k}")
    dev = torch.device("cuda:0")
    dA, dB, dD = A.to(dev), B.to(dev), D.to(dev)
    dC = C.to(dev) if C is not None else None
    dD.store.fill_(float("nan"))
    lay = {"A": Layout.make(list(A.shape), list(A.stride)), "B": Layout.make(list(B.shape), list(B.stride)),
           "D": Layout.make(list(D.shape), list(D.stride))}
    if C is not None:
        lay["C"] = Layout.make(list(C.shape), list(C.stride))
    plan = g.plan(dA.store, dB.store, dD.store, dC.store if dC is not None else None, beta, kernel=kernel,
                  tile=tile, split_k=split_k, layouts=lay, persistent=persistent)
    if expect_kernel:
        assert plan["kernel_name"] == expect_kernel, plan
    amax = torch.full((1,), -1.0, dtype=torch.float32, device=dev)   # the library must clear it
    dbias = bias.to(dev) if bias is not None else None
    g.gemm(dA.store, dB.store, dD.store, dC.store if dC is not None else None, alpha, beta, kernel=kernel,
           tile=tile, split_k=split_k, layouts=lay, bias=dbias, bias_stride=bias_stride, bias_per_row=bias_per_row,
           activation=act, amax=amax, persistent=persistent)
    torch.cuda.synchronize()
    out = datagen.Matrix(dD.store.cpu(), D.shape, D.stride)
    points = all_points(M, N)
    S, T = og.gemm_points(op(A), op(B), points)
    Dpre, Cabs = og.epilogue(S, op(C) if C is not None else None, points, alpha, beta)
    Dref, mag = og.fused_epilogue(Dpre, Cabs, points, bias, bias_stride, bias_per_row, act)
    got = og.read_points(op(out), points)
    res = og.check_fused(got, Dref, T, mag, alpha, A.dtype, act)
    written_max = float(np.nanmax(np.abs(got))) if got.size else 0.0
    say(f"[gemm-fused] {label} {plan['kernel_name']}: {res}; amax {amax.item()} vs max|D| {written_max}")
    return res, plan, float(amax.item()), written_max
