"""Fused epilogue on the GPU ("CUTLASS, in depth", "Epilogue fusion"):
D = act(alpha*A*B + beta*C + bias) and max |D| from every kernel family,
checked output by output against the oracle (the GEMM bound carried through
the activation's Lipschitz constant), and the reported maximum equal to the
maximum of the written output exactly."""

import pytest
import torch

import datagen
from tests.gemm_cases import run_and_check_fused

pytestmark = pytest.mark.gpu

F16, BF16 = torch.float16, torch.bfloat16


def _pad8(x):
    return (x + 7) // 8 * 8


def _case(M, N, K, dtype, a_major, b_major, d_major, beta, seed, dist="uniform"):
    A = datagen.matrix(M, K, dtype, a_major, dist, seed, ld=_pad8(K if a_major == "row" else M), k_for_scale=K)
    B = datagen.matrix(K, N, dtype, b_major, dist, seed + 1, ld=_pad8(N if b_major == "row" else K), k_for_scale=K)
    ldd = _pad8(N if d_major == "row" else M)
    C = datagen.matrix(M, N, dtype, d_major, "uniform", seed + 2, ld=ldd) if beta != 0 else None
    D = datagen.zeros(M, N, dtype, d_major, ld=ldd)
    return A, B, C, D


def _bias(n, dtype, seed, stride=1):
    g = torch.Generator().manual_seed(seed)
    return (torch.rand(n * stride, generator=g, dtype=torch.float64) * 2 - 1).to(dtype)


CASES = [
    # (label, M, N, K, dtype, a, b, d, beta, kernel, split_k, expect, block tile)
    ("wave16", 250, 130, 72, F16, "row", "col", "row", 0.5, "auto", 0, "wave16", None),
    ("tiled", 512, 512, 256, BF16, "row", "col", "row", 0.0, "auto", 0, "tiled", None),
    ("tiled-256", 512, 512, 256, F16, "row", "col", "row", 0.5, "tiled", 1, "tiled", (256, 256)),
    ("tiled-ragged", 300, 520, 200, F16, "row", "col", "row", -1.0, "tiled", 0, "tiled", None),
    ("tiled-ragged-256", 300, 520, 200, BF16, "row", "col", "row", 1.0, "tiled", 0, "tiled", (256, 256)),
    ("tiled-mn", 264, 392, 96, BF16, "col", "row", "row", 1.0, "tiled", 0, "tiled", None),
    ("tiled-mn-256", 264, 392, 96, F16, "col", "row", "row", 0.0, "tiled", 0, "tiled", (256, 256)),
    ("tiled-split", 512, 768, 512, BF16, "row", "col", "row", 0.5, "tiled", 2, "tiled", None),
    ("tiled-128", 392, 648, 192, F16, "col", "col", "row", 0.5, "tiled", 1, "tiled", (128, 128)),
    ("skinny", 32, 1024, 4096, BF16, "row", "col", "row", 0.0, "auto", 0, "skinny", None),
    ("skinny-split", 17, 512, 4096, F16, "row", "col", "row", 0.5, "auto", 2, "skinny", None),
]


@pytest.mark.parametrize("act", [None, "relu", "gelu"])
@pytest.mark.parametrize("per_row", [False, True])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_epilogue_all_kernels(case, per_row, act):
    label, M, N, K, dtype, a, b, d, beta, kernel, split, expect, tile = case
    A, B, C, D = _case(M, N, K, dtype, a, b, d, beta, seed=M + N + K)
    bias = _bias(M if per_row else N, dtype, seed=K)
    res, plan, amax, wmax = run_and_check_fused(A, B, C, D, 1.5, beta, bias, per_row, act, kernel=kernel,
                                                split_k=split, expect_kernel=expect, label=label, tile=tile)
    if tile:
        assert (plan["tile_m"], plan["tile_n"]) == tile
    assert res.ok, str(res)
    assert amax == wmax


def test_fused_epilogue_transposed_output_and_strided_bias():
    """An M-major D is solved as D^T = B^T A^T: a bias along D's rows becomes
    one along the kernel's columns; the bias is read with a stride."""
    A, B, C, D = _case(512, 256, 128, BF16, "row", "col", "col", 0.5, seed=9)
    for per_row in (True, False):
        bias = _bias(512 if per_row else 256, BF16, seed=10, stride=3)
        res, plan, amax, wmax = run_and_check_fused(A, B, C, D, 1.0, 0.5, bias, per_row, "gelu", bias_stride=3,
                                                    expect_kernel="tiled", label="d-col-major")
        assert res.ok, str(res)
        assert amax == wmax


def test_amax_alone_and_relu_without_bias():
    A, B, C, D = _case(256, 256, 64, F16, "row", "col", "row", 0.0, seed=12, dist="normal")
    res, _, amax, wmax = run_and_check_fused(A, B, None, D, 1.0, 0.0, None, False, None, label="amax-only")
    assert res.ok and amax == wmax > 0
    res, _, amax, wmax = run_and_check_fused(A, B, None, D, -1.0, 0.0, None, False, "relu", label="relu")
    assert res.ok and amax == wmax
