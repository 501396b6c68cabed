"""The allocation-free entry point (lt_gemm_run_noalloc) on the GPU, through
the C ABI: on plans whose kernels use scratch (the split-K partials and
arrival counters of the tiled split remainder, the skinny kernel's split-K
partials), its output is checked against the oracle and against the output of
lt_gemm_run_ex on the same inputs, on two calls in a row, the second with a
smaller input, so the second call runs on the array the first one left
behind."""

import pytest
import torch

import datagen
from tests.gemm_cases import all_points, check_points, op, say
from oracle import gemm as og

pytestmark = pytest.mark.gpu

BF16, F16 = torch.bfloat16, torch.float16


def _case(M, N, K, dtype, beta, seed):
    A = datagen.matrix(M, K, dtype, "row", "uniform", seed)
    B = datagen.matrix(K, N, dtype, "col", "uniform", seed + 1)
    C = datagen.matrix(M, N, dtype, "row", "uniform", seed + 2) if beta != 0 else None
    D = datagen.zeros(M, N, dtype, "row")
    return A, B, C, D


def _run_both(A, B, C, D, alpha, beta, split, label, **epi):
    """(plan, output of lt_gemm_run_ex, output of lt_gemm_run_noalloc)."""
    from layout_algebra_tiled_amd import gemm as g
    say(f"[noalloc] {label} M={D.shape[0]} N={D.shape[1]} K={A.shape[1]} split_k={split}")
    dev = torch.device("cuda:0")
    dA, dB = A.to(dev), B.to(dev)
    dC = C.to(dev).view() if C is not None else None
    outs = []
    for fn in (g.gemm, g.gemm_noalloc):
        dD = D.to(dev)
        dD.store.fill_(float("nan"))
        fn(dA.view(), dB.view(), dD.view(), dC, alpha, beta, split_k=split, **epi)
        torch.cuda.synchronize()
        outs.append(datagen.Matrix(dD.store.cpu(), D.shape, D.stride))
    plan = g.plan(dA.view(), dB.view(), D.to(dev).view(), dC, beta, split_k=split)
    return plan, outs[0], outs[1]


def _check(A, B, C, out, alpha, beta, label):
    M, N = out.shape
    res = check_points(A, B, C, out, alpha, beta, all_points(M, N))
    say(f"[noalloc] {label}: {res}")
    assert res.ok, str(res)


@pytest.mark.parametrize("shapes", [
    # tiled split remainder: 16 tiles x 4 segments (16 MiB of partials), then 6 tiles x 2
    [(1024, 1024, 2048, BF16, 0.0, 4), (512, 768, 512, F16, 0.5, 2)],
    # skinny split-K: 4 K segments, then 2
    [(32, 1024, 8192, BF16, 0.0, 4), (17, 512, 4096, F16, 0.5, 2)],
])
def test_noalloc_matches_run_ex_twice_in_a_row(shapes):
    for i, (M, N, K, dt, beta, split) in enumerate(shapes):
        A, B, C, D = _case(M, N, K, dt, beta, seed=100 * i + M)
        plan, ex, na = _run_both(A, B, C, D, 1.0, beta, split, f"call {i + 1}")
        assert plan["workspace_bytes"] > 0, plan   # the plan really uses scratch
        _check(A, B, C, ex, 1.0, beta, f"call {i + 1} run_ex")
        _check(A, B, C, na, 1.0, beta, f"call {i + 1} noalloc")
        # same kernels, same inputs: only the split fix-up's summation order
        # may differ, so the two outputs agree to the same bound
        pts = all_points(M, N)
        S, T = og.gemm_points(op(A), op(B), pts)
        Dref, Cabs = og.epilogue(S, op(C) if C is not None else None, pts, 1.0, beta)
        b = og.bound(T, Cabs, Dref, 1.0, dt)
        diff = abs(og.read_points(op(ex), pts) - og.read_points(op(na), pts))
        assert (diff <= b).all()


def test_noalloc_fused_epilogue_and_amax():
    """The fused epilogue through the allocation-free call: bias, GELU and
    max |D| on a split-remainder plan."""
    M, N, K = 1024, 1024, 2048
    A, B, C, D = _case(M, N, K, BF16, 0.0, seed=7)
    bias = (torch.arange(N, dtype=torch.float64) / N - 0.5).to(BF16)
    from layout_algebra_tiled_amd import gemm as g
    dA, dB = A.to("cuda"), B.to("cuda")
    dD = D.to("cuda")
    dD.store.fill_(float("nan"))
    amax = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    g.gemm_noalloc(dA.view(), dB.view(), dD.view(), None, 1.0, 0.0, split_k=4, bias=bias.cuda(), activation="gelu",
                   amax=amax)
    torch.cuda.synchronize()
    out = datagen.Matrix(dD.store.cpu(), D.shape, D.stride)
    pts = all_points(M, N)
    S, T = og.gemm_points(op(A), op(B), pts)
    Dpre, Cabs = og.epilogue(S, None, pts, 1.0, 0.0)
    Dref, mag = og.fused_epilogue(Dpre, Cabs, pts, bias, 1, False, "gelu")
    got = og.read_points(op(out), pts)
    res = og.check_fused(got, Dref, T, mag, 1.0, BF16, "gelu")
    say(f"[noalloc] fused: {res}; amax {amax.item()}")
    assert res.ok, str(res)
    assert amax.item() == float(abs(got).max())


def test_noalloc_refuses_a_plan_larger_than_its_scratch():
    """A forced split whose partials exceed the static array: refused before
    anything is launched, and the output is left untouched."""
    from layout_algebra_tiled_amd import gemm as g
    from layout_algebra_tiled_amd._lib import LtError, LT_NOALLOC_SCRATCH_BYTES
    M = N = 4096
    K = 1024
    A = torch.zeros(M, K, dtype=BF16, device="cuda")
    B = torch.zeros(N, K, dtype=BF16, device="cuda").t()
    D = torch.full((M, N), 3.0, dtype=BF16, device="cuda")
    plan = g.plan(A, B, D, None, 0.0, split_k=8)
    assert plan["workspace_bytes"] > LT_NOALLOC_SCRATCH_BYTES
    with pytest.raises(LtError) as e:
        g.gemm_noalloc(A, B, D, None, 1.0, 0.0, split_k=8)
    assert e.value.name == "LT_ERR_WORKSPACE"
    torch.cuda.synchronize()
    assert bool((D == 3.0).all())
