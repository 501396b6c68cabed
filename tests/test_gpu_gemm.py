"""GEMM parity on the GPU: the library's kernels against the fp64 oracle,
element by element, within |D - D_ref| <= 2e-3 (|alpha| sum|a b| + |beta c|)
+ one output ulp. Small cases check every output; the full-size workloads
check sampled outputs (corners, edges and random points) in the launch
configuration the benchmark times."""

import numpy as np
import pytest
import torch

import datagen
from tests.gemm_cases import (all_points, check_all_rows, check_points, op, run_and_check, run_gemm,
                              sample_points, say)
from oracle import gemm as og

pytestmark = pytest.mark.gpu

F16, BF16 = torch.float16, torch.bfloat16


def _pad8(x):
    return (x + 7) // 8 * 8


def _case(M, N, K, dtype, a_major, b_major, d_major, alpha, beta, dist="uniform", seed=0, lds=None):
    """Leading dimensions default to the extent rounded up to 8 elements (the
    128-bit alignment rule); padding holds NaN."""
    if lds is None:
        lds = (_pad8(K if a_major == "row" else M), _pad8(N if b_major == "row" else K),
               _pad8(N if d_major == "row" else M))
    A = datagen.matrix(M, K, dtype, a_major, dist, seed + 0, ld=lds[0], k_for_scale=K)
    B = datagen.matrix(K, N, dtype, b_major, dist, seed + 1, ld=lds[1], k_for_scale=K)
    C = datagen.matrix(M, N, dtype, d_major, "uniform", seed + 2, ld=lds[2]) if beta != 0 else None
    D = datagen.zeros(M, N, dtype, d_major, ld=lds[2])
    return A, B, C, D


def _ok(res):
    assert res.ok, str(res)


# ---------------------------------------------------------------------------
# the small workload: 256x128x64 fp16 tiled 16x16 by zipped_divide
# ---------------------------------------------------------------------------

def test_workload_256x128x64_all_outputs():
    c = datagen.config(1)
    A, B, C, D = c.make()
    res, plan, _ = run_and_check(A, B, None, D, c.alpha, c.beta, expect_kernel="wave16", label="cfg1")
    _ok(res)
    assert res.n == 256 * 128 and (plan["tile_m"], plan["tile_n"]) == (16, 16)


# ---------------------------------------------------------------------------
# the 256x256 tiled kernel, every output checked
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K,dtype,beta,dist", [
    (512, 512, 512, F16, 0.5, "uniform"),
    (512, 768, 1024, BF16, 0.0, "normal_over_sqrtk"),
    (256, 256, 64, BF16, 1.0, "uniform"),
    (768, 512, 192, F16, -1.0, "uniform"),
])
def test_tiled_all_outputs(M, N, K, dtype, beta, dist):
    A, B, C, D = _case(M, N, K, dtype, "row", "col", "row", 1.0, beta, dist, seed=100 + K)
    res, _, _ = run_and_check(A, B, C, D, 1.0, beta, expect_kernel="tiled", label="tiled")
    _ok(res)


def test_tiled_padded_leading_dimensions():
    """Leading dimensions larger than the extents (padding holds NaN)."""
    M, N, K = 512, 256, 128
    A, B, C, D = _case(M, N, K, BF16, "row", "col", "row", 1.0, 0.5, seed=7, lds=(K + 64, K + 8, N + 16))
    res, _, _ = run_and_check(A, B, C, D, 1.0, 0.5, expect_kernel="tiled", label="tiled-padded")
    _ok(res)


# ---------------------------------------------------------------------------
# ragged shapes on the 256x256 kernel: edge tiles clamp their copy rows and
# predicate their stores; a partial K slice is zero-filled (every output)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K,dtype,a_major,b_major,alpha,beta,lds", [
    (300, 520, 200, BF16, "row", "col", 1.0, 0.5, None),           # ragged M and N, K = 3*64 + 8
    (257, 258, 136, F16, "row", "col", 1.0, -1.0, (136, 136, 264)),  # N % 4 = 2: partial 4-output groups
    (512, 256, 8, BF16, "row", "col", 1.0, 0.0, None),             # a single, partial K slice
    (264, 392, 77, F16, "col", "row", 2.0, -1.0, None),            # M-/N-major operands, any K
    (520, 264, 1000, BF16, "col", "col", 1.0, 0.0, None),          # M-major A, K-major B
    (1, 300, 64, F16, "row", "col", 1.0, 0.0, None),               # one row
    (700, 9, 328, BF16, "row", "col", 1.0, 1.0, (328, 328, 16)),   # nine columns, padded D and C
])
@pytest.mark.parametrize("tile_n", [256, 128])
def test_tiled_ragged_all_outputs(M, N, K, dtype, a_major, b_major, alpha, beta, lds, tile_n):
    A, B, C, D = _case(M, N, K, dtype, a_major, b_major, "row", alpha, beta, seed=M + N + K, lds=lds)
    res, plan, _ = run_and_check(A, B, C, D, alpha, beta, kernel="tiled", tile=(256, tile_n),
                                 expect_kernel="tiled", label="tiled-ragged")
    _ok(res)
    tiles = ((M + 255) // 256) * ((N + tile_n - 1) // tile_n)
    assert plan["tile_n"] == tile_n and plan["grid"] == tiles - plan["sk_tiles"] + plan["sk_workgroups"]


@pytest.mark.parametrize("K", [64, 128, 192, 256, 320])
@pytest.mark.parametrize("a_major,b_major", [("row", "col"), ("col", "row"), ("row", "row"), ("col", "col")])
@pytest.mark.parametrize("tile_n", [256, 128])
def test_tiled_slice_counts_every_major(K, a_major, b_major, tile_n):
    """The 256x256 (2 LDS stages) and 256x128 (3 stages) kernels at 1 to 5 K
    slices (no refill, the refill loop entered or not, several refills) for
    every operand major-ness, on 4 (8) tiles, every output checked: the issue
    order of copies, fragment reads and MFMAs, and its explicit waits, differ
    between those loop shapes."""
    M, N = 512, 512
    A, B, C, D = _case(M, N, K, BF16, a_major, b_major, "row", 1.0, 0.5, seed=K + 7)
    res, plan, _ = run_and_check(A, B, C, D, 1.0, 0.5, kernel="tiled", split_k=1, tile=(256, tile_n),
                                 expect_kernel="tiled", label=f"slices {K // 64} {a_major}/{b_major} 256x{tile_n}")
    _ok(res)
    assert plan["waves"] == 4 and plan["grid"] == (512 // 256) * (512 // tile_n) and plan["tile_n"] == tile_n


# ---------------------------------------------------------------------------
# the persistent launch of 256x128 tiles: one workgroup per compute unit
# walks its tiles, copying the next tile's first slices while the current
# one finishes (every output checked)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K,dtype,a_major,b_major,alpha,beta", [
    # 320 tiles, a multiple of 8 (XCD regrouping): 8 workgroups take 2 tiles,
    # 4 K slices (the fewest the launch takes)
    (4096, 2560, 256, BF16, "row", "col", 1.0, 0.0),
    # 128 tiles: one each, 5 slices, M-/N-major operands, C loaded
    (2048, 2048, 320, F16, "col", "row", 2.0, -1.0),
    # 135 tiles, not a multiple of 8 (no regrouping)
    (2304, 1920, 256, F16, "row", "row", 1.0, 0.5),
    # 323 tiles on 256 workgroups without regrouping: 67 take two
    (4864, 2176, 512, BF16, "col", "col", 1.0, 1.0),
    # 528 tiles: 2 or 3 per workgroup; 7 slices
    (6144, 2816, 448, BF16, "row", "col", 1.0, -0.5),
    # 256 tiles, 16 slices, bf16 M-major A
    (2048, 4096, 1024, BF16, "col", "col", 0.5, 0.0),
])
def test_tiled_persistent_all_outputs(M, N, K, dtype, a_major, b_major, alpha, beta):
    A, B, C, D = _case(M, N, K, dtype, a_major, b_major, "row", alpha, beta, seed=M + K)
    res, plan, _ = run_and_check(A, B, C, D, alpha, beta, kernel="tiled", tile=(256, 128), persistent=True,
                                 expect_kernel="tiled", label="tiled-persistent")
    _ok(res)
    tiles = (M // 256) * (N // 128)
    assert plan["persistent"] == 1 and plan["grid"] == min(tiles, 256) and plan["tiles"] == tiles


@pytest.mark.parametrize("M,N,K,dtype,a_major,b_major,alpha", [
    # 320 256x256 tiles (XCD regrouping), 4 slices (the fewest)
    (5120, 4096, 256, BF16, "row", "col", 1.0),
    # 135 tiles, one each, no regrouping; M-/N-major, 5 slices
    (2304, 3840, 320, F16, "col", "row", 2.0),
    # 528 tiles: 2 or 3 per workgroup, 7 slices
    (6144, 5632, 448, BF16, "col", "col", 1.0),
    # 289 tiles without regrouping: 33 workgroups take two
    (4352, 4352, 576, F16, "row", "row", -1.0),
])
def test_tiled_persistent_256_all_outputs(M, N, K, dtype, a_major, b_major, alpha):
    """The persistent launch of 256x256 tiles (2 LDS stages; beta = 0)."""
    A, B, C, D = _case(M, N, K, dtype, a_major, b_major, "row", alpha, 0.0, seed=M + N + K)
    res, plan, _ = run_and_check(A, B, None, D, alpha, 0.0, kernel="tiled", tile=(256, 256), persistent=True,
                                 split_k=1, expect_kernel="tiled", label="tiled-persistent-256")
    _ok(res)
    tiles = (M // 256) * (N // 256)
    assert plan["persistent"] == 1 and plan["grid"] == min(tiles, 256) and plan["tiles"] == tiles


@pytest.mark.parametrize("tile_n", [128, 256])
def test_tiled_persistent_in_place_d_is_c(tile_n):
    """D == C through the persistent launch (256x128: C loaded at each
    tile's start, D stored at its end; 256x256 runs only with beta = 0, so
    there D == C is a plain overwrite with beta = 0)."""
    from layout_algebra_tiled_amd import gemm as g
    M, N, K = 2560, 2048, 256
    beta = 0.5 if tile_n == 128 else 0.0
    A, B, C, _ = _case(M, N, K, BF16, "row", "col", "row", 1.0, 0.5, seed=77)
    dA, dB, dC = A.to("cuda"), B.to("cuda"), C.to("cuda")
    p = g.plan(dA.view(), dB.view(), dC.view(), dC.view(), beta, kernel="tiled", tile=(256, tile_n),
               persistent=True, split_k=1)
    assert p["persistent"] == 1
    g.gemm(dA.view(), dB.view(), dC.view(), dC.view(), 1.0, beta, kernel="tiled", tile=(256, tile_n),
           persistent=True, split_k=1)
    torch.cuda.synchronize()
    pts = all_points(M, N)
    S, T = og.gemm_points(op(A), op(B), pts)
    Dref, Cabs = og.epilogue(S, op(C) if beta else None, pts, 1.0, beta)
    got = og.read_points(og.Operand(dC.store.cpu(), C.shape, C.stride), pts)
    _ok(og.check(got, Dref, T, Cabs, 1.0, BF16))


def test_tiled_persistent_option_with_a_fused_epilogue():
    """A fused epilogue runs one workgroup per tile even when the persistent
    launch is asked for: the result is the fused one, every output."""
    from tests.gemm_cases import run_and_check_fused
    M, N, K = 2048, 2048, 256
    A, B, C, D = _case(M, N, K, F16, "row", "col", "row", 1.0, -0.5, seed=78)
    bias = datagen.matrix(1, N, F16, "row", "uniform", 79).view().reshape(-1).contiguous()
    res, plan, amax, wmax = run_and_check_fused(A, B, C, D, 1.0, -0.5, bias, False, "gelu", kernel="tiled",
                                                 tile=(256, 128), persistent=True, label="fused-persistent")
    _ok(res)
    assert plan["persistent"] == 1 and amax == wmax


def test_tiled_persistent_matches_one_workgroup_per_tile():
    """The same problem through both launches of the 256x128 kernel: the
    same products summed in the same order, so the outputs agree bit for
    bit."""
    from tests.gemm_cases import run_gemm
    M, N, K = 4096, 2304, 512
    A, B, C, D = _case(M, N, K, BF16, "row", "col", "row", 1.0, 0.75, seed=3)
    p1, o1 = run_gemm(A, B, C, D, 1.0, 0.75, kernel="tiled", tile=(256, 128), persistent=True,
                      label="persistent")
    p0, o0 = run_gemm(A, B, C, D, 1.0, 0.75, kernel="tiled", tile=(256, 128), persistent=False,
                      label="per-tile")
    assert p1["persistent"] == 1 and p0["persistent"] == 0
    assert torch.equal(o1.store.view(torch.int16), o0.store.view(torch.int16))


def test_tiled_ragged_large_auto():
    """A ragged shape large enough for the automatic choice to take the 256x256 kernel."""
    M, N, K = 1000, 1304, 1000
    A, B, C, D = _case(M, N, K, BF16, "row", "col", "row", 1.0, 0.25, dist="normal_over_sqrtk", seed=5)
    pts = sample_points(M, N, 3000, seed=5)
    res, plan, _ = run_and_check(A, B, C, D, 1.0, 0.25, points=pts, expect_kernel="tiled", label="ragged-auto")
    _ok(res)


# ---------------------------------------------------------------------------
# split remainder: when the tiles do not fill whole rounds of the 256 CUs,
# the last round's tiles are split into K segments; the segments meet as
# fp32 partials and the one that finishes last stores the tile
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K,dtype,a_major,b_major,beta,split", [
    (512, 768, 512, BF16, "row", "col", 0.0, 2),       # forced: 6 tiles in 2 segments
    (512, 512, 640, F16, "row", "col", 0.5, 3),        # forced: segments of 3, 3 and 4 slices
    (300, 520, 200, BF16, "row", "col", -1.0, 2),      # ragged tiles, partial first slice
    (264, 392, 77, F16, "col", "row", 2.0, 2),         # M-/N-major operands
    (2048, 2048, 8192, BF16, "row", "col", 0.0, 4),    # forced: 64 tiles x 128 slices, 4 segments each
    (1024, 1024, 16384, BF16, "row", "col", 0.0, 0),   # the planner's split: 16 tiles x 256 slices, 8 segments
    (512, 512, 512, BF16, "row", "col", 1.0, 1),       # forced off: data-parallel only
])
def test_tiled_split_remainder_all_outputs(M, N, K, dtype, a_major, b_major, beta, split):
    A, B, C, D = _case(M, N, K, dtype, a_major, b_major, "row", 1.0, beta, seed=3 * M + K)
    pts = None if M * N <= 600_000 else sample_points(M, N, 20000, seed=M)
    res, plan, _ = run_and_check(A, B, C, D, 1.0, beta, kernel="tiled", split_k=split, points=pts,
                                 expect_kernel="tiled", label=f"tiled-split{split}")
    _ok(res)
    assert (plan["sk_tiles"] > 0) == (split != 1)


def test_tiled_split_remainder_repeated_runs_keep_counters_consistent():
    """Three runs in a row on one workspace, the middle one with another
    shape: the arrival counters start at zero every run."""
    from layout_algebra_tiled_amd import gemm as g
    ws = torch.full((64 << 20,), 255, dtype=torch.uint8, device="cuda")   # garbage on entry
    for (M, N, K) in ((512, 768, 512), (768, 256, 1024), (512, 768, 512)):
        A, B, C, D = _case(M, N, K, BF16, "row", "col", "row", 1.0, 0.0, seed=M + N)
        dA, dB, dD = A.to("cuda"), B.to("cuda"), D.to("cuda")
        dD.store.fill_(float("nan"))
        g.gemm(dA.view(), dB.view(), dD.view(), None, 1.0, 0.0, workspace=ws)
        torch.cuda.synchronize()
        pts = all_points(M, N)
        S, T = og.gemm_points(op(A), op(B), pts)
        Dref, Cabs = og.epilogue(S, None, pts, 1.0, 0.0)
        got = og.read_points(og.Operand(dD.store.cpu(), D.shape, D.stride), pts)
        _ok(og.check(got, Dref, T, Cabs, 1.0, BF16))


# ---------------------------------------------------------------------------
# layout variants, ragged shapes, degenerate cases (wave-per-tile kernel)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("a_major,b_major", [("row", "col"), ("col", "row"), ("row", "row"), ("col", "col")])
@pytest.mark.parametrize("dtype", [F16, BF16])
def test_any_major_ragged(a_major, b_major, dtype):
    M, N, K = 250, 130, 72
    A, B, C, D = _case(M, N, K, dtype, a_major, b_major, "row", 2.0, -1.0, seed=11)
    res, _, _ = run_and_check(A, B, C, D, 2.0, -1.0, label=f"ragged {a_major}/{b_major}")
    _ok(res)


def test_mn_major_operands_all_outputs():
    """M-major A and N-major B, alpha=2, beta=-1 (the layout-driven staging case)."""
    M, N, K = 512, 256, 384
    A, B, C, D = _case(M, N, K, F16, "col", "row", "row", 2.0, -1.0, seed=21)
    res, _, _ = run_and_check(A, B, C, D, 2.0, -1.0, label="mn-major")
    _ok(res)


def test_k_tail_not_multiple_of_chunk():
    """K = 70: the last 8-wide chunk is partial; A's padding columns hold NaN."""
    M, N, K = 64, 48, 70
    A, B, C, D = _case(M, N, K, BF16, "row", "col", "row", 1.0, 0.0, seed=31, lds=(72, 72, 48))
    res, _, _ = run_and_check(A, B, None, D, 1.0, 0.0, label="k-tail")
    _ok(res)


def test_m_major_output_is_solved_transposed():
    M, N, K = 512, 256, 128
    A, B, C, D = _case(M, N, K, BF16, "row", "col", "col", 1.0, 0.5, seed=41)
    res, plan, _ = run_and_check(A, B, C, D, 1.0, 0.5, expect_kernel="tiled", label="d-col-major")
    _ok(res)


def test_in_place_d_is_c():
    from layout_algebra_tiled_amd import gemm as g
    M, N, K = 256, 256, 128
    A, B, C, _ = _case(M, N, K, F16, "row", "col", "row", 1.0, 0.5, seed=51)
    dA, dB, dC = A.to("cuda"), B.to("cuda"), C.to("cuda")
    g.gemm(dA.view(), dB.view(), dC.view(), dC.view(), 1.0, 0.5)
    torch.cuda.synchronize()
    pts = all_points(M, N)
    S, T = og.gemm_points(op(A), op(B), pts)
    Dref, Cabs = og.epilogue(S, op(C), pts, 1.0, 0.5)
    got = og.read_points(og.Operand(dC.store.cpu(), C.shape, C.stride), pts)
    _ok(og.check(got, Dref, T, Cabs, 1.0, F16))


@pytest.mark.parametrize("M,N,K,dtype,a_major,b_major,alpha,beta,tile", [
    (1024, 1024, 1024, BF16, "row", "col", 1.0, 0.0, None),            # the planner's: 64 tiles, staged D
    (640, 384, 320, F16, "col", "row", 2.0, -1.0, (128, 128)),         # M-/N-major, C
    (300, 520, 200, F16, "row", "row", 1.0, 0.5, (128, 128)),          # ragged tiles, partial first slice
    (512, 768, 448, BF16, "col", "col", 1.0, 1.0, (128, 128)),
    (1536, 1536, 1536, F16, "row", "col", 1.0, 0.5, None),             # the planner's: 144 tiles, C
])
def test_tiled_128x128_all_outputs(M, N, K, dtype, a_major, b_major, alpha, beta, tile):
    """128x128 block tiles (4 waves of 64x64, 4 stages of 32 KiB), forced or
    the planner's choice for problems whose larger tiles leave CUs idle;
    every output checked."""
    A, B, C, D = _case(M, N, K, dtype, a_major, b_major, "row", alpha, beta, seed=M + 7 * K)
    res, plan, _ = run_and_check(A, B, C, D, alpha, beta, kernel="tiled" if tile else "auto", tile=tile,
                                 split_k=1 if tile else 0, expect_kernel="tiled", label="128x128")
    assert (plan["tile_m"], plan["tile_n"], plan["persistent"]) == (128, 128, 0), plan
    _ok(res)


@pytest.mark.parametrize("tile", [(128, 128), (256, 128), (256, 256)])
@pytest.mark.parametrize("beta", [0.0, 0.5])
def test_tiled_staged_edge_tiles_partial_chunks(tile, beta):
    """K-major operands: edge tiles store D through LDS too. N % 8 = 2 (D's
    rows padded to 16-byte multiples) leaves a 16-byte chunk that N cuts in
    every row; M cuts the last tile row. Every output checked."""
    M, N, K = 300, 522, 200
    A, B, C, D = _case(M, N, K, BF16, "row", "col", "row", 1.0, beta, seed=N + int(8 * beta), lds=(K, K, 528))
    res, plan, _ = run_and_check(A, B, C, D, 1.0, beta, kernel="tiled", tile=tile, split_k=1,
                                 expect_kernel="tiled", label="staged-edge")
    assert (plan["tile_m"], plan["tile_n"], plan["persistent"]) == (tile[0], tile[1], 0), plan
    _ok(res)


def test_tiled_128x128_planned_long_k_sampled():
    """The planner's 128x128 tiles on bf16 2048^2 x 8192 (256 tiles, one
    round, 128 slices each), sampled outputs."""
    M, N, K = 2048, 2048, 8192
    A, B, C, D = _case(M, N, K, BF16, "row", "col", "row", 1.0, 0.0, dist="normal_over_sqrtk", seed=5)
    res, plan, _ = run_and_check(A, B, C, D, 1.0, 0.0, points=sample_points(M, N, 20000, seed=3),
                                 expect_kernel="tiled", label="128x128 planned")
    assert (plan["tile_m"], plan["tile_n"], plan["grid"]) == (128, 128, 256), plan
    _ok(res)


def test_tiled_superblock_order_matches_the_raster():
    """The data-parallel launch in 16x16-tile super-blocks (forced; 16 x 32
    tiles: two blocks) computes every tile exactly as the raster order does:
    the outputs are bit-equal, and every one is within the oracle's bound."""
    M, N, K = 4096, 8192, 512
    A, B, C, D = _case(M, N, K, BF16, "row", "col", "row", 1.0, 0.0, dist="normal_over_sqrtk", seed=91)
    outs = {}
    for order in ("superblock", "raster"):
        plan, out = run_gemm(A, B, None, D, 1.0, 0.0, kernel="tiled", tile=(256, 256), split_k=1,
                             persistent=False, tile_order=order, label=f"order {order}")
        assert plan["tile_order"] == (2 if order == "superblock" else 1), plan
        outs[order] = out.view().clone()
    assert torch.equal(outs["superblock"].view(torch.int16), outs["raster"].view(torch.int16))
    res = check_all_rows(A, B, None, datagen.Matrix(outs["superblock"].reshape(-1), (M, N), (N, 1)), 1.0, 0.0)
    _ok(res)


def test_tiled_k_reversed_rounds():
    """The raster with odd rounds walking K downward (forced; 512 tiles, two
    rounds): every output within the oracle's bound, and only the second
    round's tiles may differ from the plain raster's (their sums run in the
    other order), the first round's bit-equal."""
    M, N, K = 4096, 8192, 512
    A, B, C, D = _case(M, N, K, BF16, "row", "col", "row", 1.0, 0.0, dist="normal_over_sqrtk", seed=93)
    outs = {}
    for order in ("raster_krev", "raster"):
        plan, out = run_gemm(A, B, None, D, 1.0, 0.0, kernel="tiled", tile=(256, 256), split_k=1,
                             persistent=False, tile_order=order, label=f"order {order}")
        assert plan["tile_order"] == (3 if order == "raster_krev" else 1), plan
        outs[order] = out.view().clone()
    res = check_all_rows(A, B, None, datagen.Matrix(outs["raster_krev"].reshape(-1), (M, N), (N, 1)), 1.0, 0.0)
    _ok(res)
    # workgroup w of the raster takes tile lin = (w % 8) * (512 / 8) + w / 8,
    # groups of 8 tile rows walked down, then right; workgroups w >= 256 form
    # the second round of 256 tiles (K walked downward there)
    tm, tn, gsz = M // 256, N // 256, 8 * (N // 256)
    round1 = set()
    for w in range(256, tm * tn):
        lin = (w % 8) * (tm * tn // 8) + w // 8
        grp, i = divmod(lin, gsz)
        round1.add((8 * grp + i % 8, i // 8))
    same = (outs["raster_krev"].view(torch.int16) == outs["raster"].view(torch.int16))
    for r in range(tm):
        for c in range(tn):
            tile_same = bool(same[256 * r:256 * (r + 1), 256 * c:256 * (c + 1)].all())
            assert tile_same or (r, c) in round1, (r, c)
    assert not bool(same.all())   # the second round did run reversed


def test_tiled_c_rows_at_the_staged_copy_offset_limit():
    """A whole 256x256 tile with C: the staged store copies the wave's 128 C
    rows through 32-bit byte offsets, so a C row stride of 2^24 - 64 elements
    takes that path and 2^24 + 64 the predicated one. Both check every
    output. C lives in one 8.6 GB device buffer of which only the 256 rows
    are written."""
    from layout_algebra_tiled_amd import gemm as g
    from layout_algebra_tiled_amd.layout import Layout
    M = N = 256
    K = 128
    A, B, C, D = _case(M, N, K, F16, "row", "col", "row", 1.0, 0.5, seed=77)
    dev = torch.device("cuda:0")
    dA, dB, dD = A.to(dev), B.to(dev), D.to(dev)
    big = torch.empty((M - 1) * ((1 << 24) + 64) + N, dtype=torch.float16, device=dev)
    try:
        for ldc in ((1 << 24) - 64, (1 << 24) + 64):
            say(f"[gemm] C row stride {ldc}")
            big.as_strided((M, N), (ldc, 1)).copy_(C.view().to(dev))
            dD.store.fill_(float("nan"))
            lay = {"A": Layout.make([M, K], list(A.stride)), "B": Layout.make([K, N], list(B.stride)),
                   "D": Layout.make([M, N], list(D.stride)), "C": Layout.make([M, N], [ldc, 1])}
            plan = g.plan(dA.store, dB.store, dD.store, big, 0.5, kernel="tiled", tile=(256, 256), split_k=1,
                          layouts=lay)
            assert (plan["tile_n"], plan["grid"], plan["persistent"]) == (256, 1, 0), plan
            g.gemm(dA.store, dB.store, dD.store, big, 1.0, 0.5, kernel="tiled", tile=(256, 256), split_k=1,
                   layouts=lay)
            torch.cuda.synchronize()
            out = datagen.Matrix(dD.store.cpu(), D.shape, D.stride)
            res = check_points(A, B, C, out, 1.0, 0.5, all_points(M, N))
            say(f"[gemm] C row stride {ldc}: {res}")
            _ok(res)
    finally:
        del big
        torch.cuda.empty_cache()


def test_k_zero_gives_beta_c_and_m_zero_is_noop():
    from layout_algebra_tiled_amd import gemm as g
    from layout_algebra_tiled_amd.layout import Layout
    M, N = 64, 32
    C = datagen.matrix(M, N, F16, "row", "uniform", 61).to("cuda")
    D = torch.full((M, N), float("nan"), dtype=F16, device="cuda")
    a = torch.empty(64, dtype=F16, device="cuda")
    b = torch.empty(64, dtype=F16, device="cuda")
    g.gemm(a, b, D, C.view(), 1.0, 0.5,
           layouts={"A": Layout.make([M, 0], [8, 1]), "B": Layout.make([0, N], [1, 8])})
    torch.cuda.synchronize()
    want = (0.5 * C.view().float()).to(F16)
    assert torch.equal(D.cpu(), want.cpu())
    E = torch.full((8,), 7.0, dtype=F16, device="cuda")
    g.gemm(a, b, E, None, 1.0, 0.0, layouts={"A": Layout.make([0, 8], [8, 1]), "B": Layout.make([8, 1], [1, 8]),
                                           "D": Layout.make([0, 1], [8, 1])})
    torch.cuda.synchronize()
    assert torch.all(E.cpu() == 7.0)


def test_two_calls_in_a_row_different_sizes():
    for (M, N, K) in ((512, 512, 256), (256, 256, 64)):
        A, B, C, D = _case(M, N, K, BF16, "row", "col", "row", 1.0, 0.0, seed=M + K)
        res, _, _ = run_and_check(A, B, None, D, 1.0, 0.0, label="repeat")
        _ok(res)


# ---------------------------------------------------------------------------
# skinny (M <= 32) kernel
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K,split", [(32, 1024, 4096, 0), (17, 512, 4096, 1), (17, 512, 4096, 2),
                                         (32, 256, 2048, 4), (1, 64, 512, 1), (32, 64, 256, 1),
                                         (8, 128, 3072, 3),
                                         # 18 256-deep slots (3 steady trips of the 4-slot ring, 6 drained)
                                         (32, 256, 4608, 1),
                                         # 19 slots: 4 steady trips, 3 drained
                                         (20, 512, 4864, 1),
                                         # 64 slots, 15 steady trips
                                         (31, 96, 16384, 1)])
def test_skinny_all_outputs(M, N, K, split):
    A, B, C, D = _case(M, N, K, BF16, "row", "col", "row", 1.0, 0.0, dist="normal", seed=71)
    res, plan, _ = run_and_check(A, B, None, D, 1.0, 0.0, split_k=split, expect_kernel="skinny", label="skinny")
    _ok(res)
    if split:
        assert plan["split_k"] == split


def test_skinny_with_beta():
    A, B, C, D = _case(32, 512, 1024, F16, "row", "col", "row", 0.5, 2.0, seed=81)
    res, _, _ = run_and_check(A, B, C, D, 0.5, 2.0, expect_kernel="skinny", label="skinny-beta")
    _ok(res)


# ---------------------------------------------------------------------------
# more tiles than CUs (several rounds of one workgroup per tile; the
# persistent launch has tests of its own), every output: K-major and M/N-major,
# partial first slices, fewer slices than stages, ragged edges, beta != 0,
# tile counts with and without the per-XCD regrouping of workgroups
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K,dtype,a_major,b_major,alpha,beta,tile_n", [
    (4096, 4096, 192, BF16, "row", "col", 1.0, 0.0, 128),    # 512 tiles: two rounds
    (4352, 4096, 200, F16, "col", "row", 1.0, 0.5, 256),     # 272 tiles; partial first slice
    (4096, 8192, 64, BF16, "row", "col", 1.0, 0.0, 256),     # one slice per tile (fewer than the stages)
    (6144, 4096, 256, F16, "col", "row", 2.0, -1.0, 128),    # M-/N-major, 768 tiles, C read
    (4100, 4104, 192, BF16, "row", "row", 1.0, 0.5, 128),    # 561 ragged tiles, no XCD regrouping
    (4104, 4112, 192, F16, "col", "col", 1.0, 0.0, 256),     # 289 ragged tiles of 256x256
    # 256x128 tiles with beta != 0: the C tile staged through LDS during the
    # last slices (interior tiles), exactly three slices, a partial first
    # slice, ragged edge tiles that read C from global memory
    (4608, 3584, 192, F16, "row", "col", 1.0, 0.5, 128),     # 504 tiles, 3 slices
    (4608, 3584, 200, BF16, "col", "row", -1.5, 2.0, 128),   # 4 slices, the first partial
    (4100, 4104, 320, F16, "row", "row", 1.0, -1.0, 128),    # ragged: edge tiles read C directly
    # K-major: edge tiles store D through LDS, whole tiles copy C through it
    (4100, 4104, 256, BF16, "row", "col", 1.0, 0.5, 256),    # 289 tiles
    (4100, 4104, 256, F16, "row", "col", 1.0, -1.0, 128),    # 561 tiles, C in the accumulators' layout
])
def test_many_rounds_tiled_all_outputs(M, N, K, dtype, a_major, b_major, alpha, beta, tile_n):
    A, B, C, D = _case(M, N, K, dtype, a_major, b_major, "row", alpha, beta, seed=M + K + tile_n)
    plan, out = run_gemm(A, B, C, D, alpha, beta, kernel="tiled", split_k=1, tile=(256, tile_n),
                         expect_kernel="tiled", label=f"rounds 256x{tile_n}", persistent=False)
    tiles = ((M + 255) // 256) * ((N + tile_n - 1) // tile_n)
    assert plan["tiles"] == plan["grid"] == tiles > 256, plan
    res = check_all_rows(A, B, C, out, alpha, beta)
    say(f"[gemm] rounds {M}x{N}x{K} 256x{tile_n}: {res}")
    _ok(res)


# ---------------------------------------------------------------------------
# the full-size workloads, every output, benchmark launch configuration
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg,kernel,tile_n", [(2, "tiled", 256), (3, "tiled", 256), (4, "tiled", 128),
                                                (5, "skinny", None)])
def test_full_size_workloads_every_output(cfg, kernel, tile_n):
    """The benchmark's workloads at full size, in the launch configuration
    the benchmark times (the automatic plan), every output checked against
    the oracle: at these sizes the XCD regrouping of workgroups and the
    raster groups past the first are in play."""
    c = datagen.config(cfg)
    say(f"[gemm] generating inputs of workload {cfg}: {c.name}")
    A, B, C, D = c.make()
    C = C if c.beta != 0 else None
    plan, out = run_gemm(A, B, C, D, c.alpha, c.beta, expect_kernel=kernel, label=f"cfg{cfg}")
    if tile_n:
        assert plan["tile_n"] == tile_n, plan
    res = check_all_rows(A, B, C, out, c.alpha, c.beta)
    say(f"[gemm] cfg{cfg}: {res}")
    _ok(res)
    assert res.n == c.M * c.N
