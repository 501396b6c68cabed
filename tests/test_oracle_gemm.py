"""Pins for the GEMM oracle and its error bound, plus planted-mistake checks
that show the pins catch a wrong oracle. Everything here runs on the CPU."""

import ctypes
import os
import subprocess

from tests.proc import skip_if_gpu_initialised

import numpy as np
import pytest
import torch

import datagen
from oracle import gemm as og
from oracle import layout as ol


def _op(m: datagen.Matrix) -> og.Operand:
    return og.Operand(m.store, m.shape, m.stride)


def _dense(m: datagen.Matrix) -> np.ndarray:
    return m.view().to(torch.float64).numpy()


def _all_points(M, N):
    return np.array([(i, j) for i in range(M) for j in range(N)], dtype=np.int64)


@pytest.fixture(scope="module", autouse=True)
def _built():
    og.build()


def test_identity_a_gives_b():
    """A = I: the sum has one nonzero term, so S == B exactly and
    D_ref == alpha*B + beta*C in two roundings."""
    M = K = 24
    N = 17
    A = datagen.place(np.eye(M), torch.float16, "row")
    B = datagen.matrix(K, N, torch.float16, "col", "uniform", 11)
    C = datagen.matrix(M, N, torch.float16, "row", "uniform", 12)
    ij = _all_points(M, N)
    S, T = og.gemm_points(_op(A), _op(B), ij)
    b = _dense(B).reshape(-1)
    assert np.array_equal(S, b) and np.array_equal(T, np.abs(b))
    Dref, Cabs = og.epilogue(S, _op(C), ij, 2.0, -0.5)
    c = _dense(C).reshape(-1)
    assert np.array_equal(Dref, 2.0 * b + -0.5 * c)
    assert np.array_equal(Cabs, np.abs(-0.5 * c))


def test_small_integers_exact_against_python_ints():
    """Entries in {-2..2}: every partial sum is an exact small integer, so the
    oracle must equal a brute-force sum over Python ints."""
    M, N, K = 9, 7, 64
    A = datagen.matrix(M, K, torch.bfloat16, "row", "smallint", 21)
    B = datagen.matrix(K, N, torch.bfloat16, "row", "smallint", 22)
    a = [[int(v) for v in row] for row in _dense(A)]
    b = [[int(v) for v in row] for row in _dense(B)]
    S, T = og.gemm_rows(_op(A), _op(B), range(M))
    for i in range(M):
        for j in range(N):
            assert S[i, j] == sum(a[i][k] * b[k][j] for k in range(K))
            assert T[i, j] == sum(abs(a[i][k] * b[k][j]) for k in range(K))


@pytest.mark.parametrize("a_major,b_major", [("row", "col"), ("col", "row"), ("row", "row"), ("col", "col")])
def test_matches_numpy_matmul_any_layout(a_major, b_major):
    """Library routine cross-check (float64 matmul) on a non-square shape,
    with operands stored through different layouts (and padded leading
    dimensions) — a transposed operand or a dropped term would fail this."""
    M, N, K = 37, 53, 29
    A = datagen.matrix(M, K, torch.float16, a_major, "uniform", 31, ld=(K + 3 if a_major == "row" else M + 5))
    B = datagen.matrix(K, N, torch.float16, b_major, "uniform", 32, ld=(N + 2 if b_major == "row" else K + 7))
    S, T = og.gemm_rows(_op(A), _op(B), range(M))
    a, b = _dense(A), _dense(B)
    assert np.allclose(S, a @ b, rtol=0, atol=1e-12)
    assert np.allclose(T, np.abs(a) @ np.abs(b), rtol=0, atol=1e-12)


def test_points_equal_rows():
    M, N, K = 16, 12, 40
    A = datagen.matrix(M, K, torch.bfloat16, "col", "normal", 41)
    B = datagen.matrix(K, N, torch.bfloat16, "row", "normal", 42)
    S1, T1 = og.gemm_rows(_op(A), _op(B), range(M))
    S2, T2 = og.gemm_points(_op(A), _op(B), _all_points(M, N))
    assert np.array_equal(S1.reshape(-1), S2) and np.array_equal(T1.reshape(-1), T2)


def test_beta_zero_never_reads_c():
    M, N, K = 4, 4, 8
    A = datagen.matrix(M, K, torch.float16, "row", "uniform", 1)
    B = datagen.matrix(K, N, torch.float16, "col", "uniform", 2)
    C = datagen.place(np.full((M, N), np.nan), torch.float16, "row")
    ij = _all_points(M, N)
    S, _ = og.gemm_points(_op(A), _op(B), ij)
    Dref, Cabs = og.epilogue(S, _op(C), ij, 1.0, 0.0)
    assert np.all(np.isfinite(Dref)) and np.all(Cabs == 0)


def test_empty_k_gives_beta_c():
    M, N = 3, 5
    A = datagen.place(np.zeros((M, 0)), torch.float16, "row")
    B = datagen.place(np.zeros((0, N)), torch.float16, "col")
    C = datagen.matrix(M, N, torch.float16, "row", "uniform", 3)
    ij = _all_points(M, N)
    S, T = og.gemm_points(_op(A), _op(B), ij)
    assert np.all(S == 0) and np.all(T == 0)
    Dref, _ = og.epilogue(S, _op(C), ij, 1.0, 0.5)
    assert np.array_equal(Dref, 0.5 * _dense(C).reshape(-1))


# ---------------------------------------------------------------------------
# ulp_out and the bound
# ---------------------------------------------------------------------------

def test_ulp_out_fp16_matches_numpy_spacing():
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.uniform(-70000, 70000, 2000), rng.uniform(-1e-3, 1e-3, 2000),
                           [1.0, 2.0, 0.5, 6.1e-5, 6.0e-5, 1e-7, 65504.0, -1.0]])
    with np.errstate(over="ignore"):
        v16 = vals.astype(np.float16)
        v16 = v16[np.isfinite(v16) & (np.abs(v16) < np.float16(65504))]
        want = np.abs(np.spacing(np.abs(v16))).astype(np.float64)
    got = og.ulp_out(v16.astype(np.float64), torch.float16)
    assert np.array_equal(got, want)
    assert og.ulp_out(np.array([0.0]), torch.float16)[0] == 2.0 ** -24


def test_ulp_out_bf16_matches_bit_increment():
    rng = np.random.default_rng(1)
    vals = torch.from_numpy(np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000),
                                            [1.0, 3.0, 2.0 ** -126, 2.0 ** -130]])).to(torch.bfloat16).abs()
    vals = vals[(vals > 0) & torch.isfinite(vals)]
    bits = vals.view(torch.int16)
    nxt = (bits + 1).view(torch.bfloat16)
    want = (nxt.to(torch.float64) - vals.to(torch.float64)).numpy()
    ok = np.isfinite(want)
    got = og.ulp_out(vals.to(torch.float64).numpy(), torch.bfloat16)
    assert np.array_equal(got[ok], want[ok])
    assert og.ulp_out(np.array([0.0]), torch.bfloat16)[0] == 2.0 ** -133


def test_check_accepts_inside_rejects_outside():
    Dref = np.array([1.0, -2.0, 0.0, 100.0])
    T = np.array([10.0, 3.0, 0.0, 50.0])
    Cabs = np.zeros(4)
    b = og.bound(T, Cabs, Dref, 1.0, torch.float16)
    assert og.check(Dref + 0.99 * b, Dref, T, Cabs, 1.0, torch.float16).ok
    r = og.check(Dref + 1.01 * b, Dref, T, Cabs, 1.0, torch.float16)
    assert not r.ok and r.n_bad == 4 and r.worst_fraction > 1.0
    bad = Dref.copy()
    bad[2] = np.nan
    assert not og.check(bad, Dref, T, Cabs, 1.0, torch.float16).ok


# ---------------------------------------------------------------------------
# Planted mistakes: each mutant of the oracle must fail a pin above.
# ---------------------------------------------------------------------------

_C_MUTANTS = {
    "drop_last_k": ("k < K; ++k", "k < K - 1; ++k"),
    "wrong_sign": ("s += p;", "s -= p;"),
    "transposed_b": ("B[k * sb0 + j * sb1]", "B[j * sb0 + k * sb1]"),
    "abs_missing": ("t += fabs(p);", "t += p;"),
}


@pytest.mark.parametrize("name", sorted(_C_MUTANTS))
def test_c_mutant_is_caught(name, tmp_path):
    skip_if_gpu_initialised()
    src = open(os.path.join(os.path.dirname(og.__file__), "gemm_oracle.c")).read()
    old, new = _C_MUTANTS[name]
    assert old in src
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", str(so), str(mpath), "-lm"])
    saved = og._lib
    try:
        og._lib = None
        lib = ctypes.CDLL(str(so))
        d, i64 = ctypes.POINTER(ctypes.c_double), ctypes.c_int64
        lib.oracle_gemm_rows.argtypes = [d, i64, i64, d, i64, i64, i64, i64, ctypes.POINTER(i64), i64, d, d]
        lib.oracle_gemm_points.argtypes = [d, i64, i64, d, i64, i64, i64, ctypes.POINTER(i64), i64, d, d]
        lib.oracle_epilogue_points.argtypes = [d, d, i64, i64, ctypes.POINTER(i64), i64,
                                               ctypes.c_double, ctypes.c_double, d, d]
        og._lib = lib
        with pytest.raises(AssertionError):
            test_matches_numpy_matmul_any_layout("row", "col")
    finally:
        og._lib = saved


def _rowmajor_unravel(shape, x):
    c = []
    for s in reversed(ol.flatten(shape)):
        c.append(x % s)
        x //= s
    return list(reversed(c))


def _bad_coalesce(L):
    pairs = [(s, d) for s, d in zip(ol.flatten(L.shape), ol.flatten(L.stride)) if s != 1]
    out = []
    for s, d in pairs:
        if out and d == out[-1][0]:          # forgets the stride factor
            out[-1] = (out[-1][0] * s, out[-1][1])
        else:
            out.append((s, d))
    return ol._from_leaves(out) if out else ol.Layout(1, 0)


def _bad_complement(B, M):
    pairs = sorted((d, s) for s, d in zip(ol.flatten(B.shape), ol.flatten(B.stride)) if d > 0 and s > 1)
    out, cur = [], 1
    for d, s in pairs:
        out.append((d // cur, cur))
        cur = s * d
    return ol.coalesce(ol._from_leaves(out or [(1, 0)]))   # drops the last leaf


@pytest.mark.parametrize("target,mutant", [
    ("unravel", _rowmajor_unravel),
    ("coalesce", _bad_coalesce),
    ("complement", _bad_complement),
])
def test_layout_mutant_is_caught(monkeypatch, target, mutant):
    import tests.test_oracle_layout as T
    monkeypatch.setattr(ol, target, mutant)
    pins = [T.test_zipped_divide_printed_form_and_modes, T.test_zipped_divide_element_37_44,
            T.test_composition_worked_example, T.test_unravel_4x3, T.test_packed_panel,
            T.test_nested_2x4_and_coalesce, T.test_costume_24, T.test_divides,
            T.test_coalesce_preserves_function_and_is_maximal,
            T.test_complement_closed_form_equals_greedy_definition]
    failures = 0
    for pin in pins:
        try:
            pin()
        except Exception:
            failures += 1
    assert failures > 0


# ---------------------------------------------------------------------------
# Fused epilogue: activation definitions pinned to values they must take
# ---------------------------------------------------------------------------

# The standard normal CDF at 1, 2 and -0.5, as printed in normal tables
# (a source other than the oracle's erf): GELU(x) = x Phi(x).
_PHI = {1.0: 0.8413447460685429, 2.0: 0.9772498680518208, -0.5: 0.3085375387259869}


def test_gelu_matches_normal_table_values():
    for x, phi in _PHI.items():
        assert abs(og.activation(np.array([x]), "gelu")[0] - x * phi) < 1e-15


def test_gelu_odd_part_is_identity_and_limits():
    """Phi(x) + Phi(-x) = 1 gives GELU(x) - GELU(-x) = x; GELU(0) = 0; far
    out GELU(x) is x on the right and 0 on the left."""
    x = np.random.default_rng(3).uniform(-6, 6, 1000)
    assert np.allclose(og.activation(x, "gelu") - og.activation(-x, "gelu"), x, rtol=0, atol=1e-13)
    assert og.activation(np.array([0.0]), "gelu")[0] == 0.0
    assert abs(og.activation(np.array([12.0]), "gelu")[0] - 12.0) < 1e-12
    assert abs(og.activation(np.array([-12.0]), "gelu")[0]) < 1e-12


def test_gelu_lipschitz_constant_bounds_the_slope():
    x = np.linspace(-8, 8, 200001)
    y = og.activation(x, "gelu")
    slope = np.abs(np.diff(y) / np.diff(x))
    assert slope.max() <= og.LIPSCHITZ["gelu"] and slope.max() > 1.12


def test_relu_and_none():
    x = np.array([-2.0, -0.0, 0.0, 0.5, 3.0])
    assert list(og.activation(x, "relu")) == [0.0, 0.0, 0.0, 0.5, 3.0]
    assert list(og.activation(x, None)) == list(x)


def test_gelu_without_sqrt2_is_caught(monkeypatch):
    """Planted mistake: erf(x) instead of erf(x / sqrt 2) misses the table."""
    monkeypatch.setattr(og, "activation", lambda x, act: x * 0.5 * (1.0 + og._erf(np.asarray(x))))
    assert any(abs(og.activation(np.array([x]), "gelu")[0] - x * phi) > 1e-6 for x, phi in _PHI.items())


def test_fused_epilogue_bias_rows_and_columns():
    ij = np.array([[0, 0], [1, 2], [3, 1]])
    pre = np.array([1.0, -2.0, 0.25])
    bias = torch.tensor([10.0, 20.0, 30.0, 40.0], dtype=torch.float16)
    d, mag = og.fused_epilogue(pre, np.zeros(3), ij, bias, 1, False, None)
    assert list(d) == [11.0, 28.0, 20.25] and list(mag) == [10.0, 30.0, 20.0]
    d, _ = og.fused_epilogue(pre, np.zeros(3), ij, bias, 1, True, "relu")
    assert list(d) == [11.0, 18.0, 40.25]
    strided = torch.tensor([10.0, 0.0, 20.0, 0.0, 30.0, 0.0, 40.0, 0.0], dtype=torch.float16)
    d, _ = og.fused_epilogue(pre, np.zeros(3), ij, strided, 2, False, None)   # every other value
    assert list(d) == [11.0, 28.0, 20.25]


# ---------------------------------------------------------------------------
# The tolerance itself: bound() and check_fused() against budgets worked out
# by hand from the stated bound
#   |D - D_ref| <= 2e-3 * (|alpha| * sum_k |a b| + |beta c|) + one output ulp
# (and, through an activation, that budget times its Lipschitz constant),
# never through the functions under test. Planted mutants of the oracle's
# source must each fail one of these pins.
# ---------------------------------------------------------------------------

# (dtype, alpha, T, |beta c|, D_ref, budget)
_BOUND_CASES = [
    # fp16, alpha 2, T 10, |beta c| 0.5 at D_ref 1: 2e-3 * 20.5 + 2^-10
    (torch.float16, 2.0, 10.0, 0.5, 1.0, 0.041 + 2.0 ** -10),
    # a negative alpha counts by its magnitude; ulp of 5 in fp16 is 2^(2-10)
    (torch.float16, -3.0, 4.0, 0.0, -5.0, 0.024 + 2.0 ** -8),
    # fp16 below the smallest normal (2^-14): the subnormal spacing 2^-24
    (torch.float16, 1.0, 0.0, 0.0, 6.0e-5, 2.0 ** -24),
    # bf16 at D_ref = 0 with nothing summed: the 2^-133 floor
    (torch.bfloat16, 1.0, 0.0, 0.0, 0.0, 2.0 ** -133),
    # bf16 at 3: 2e-3 * (0.5 * 8 + 1) + 2^(1-7)
    (torch.bfloat16, 0.5, 8.0, 1.0, 3.0, 0.01 + 2.0 ** -6),
    # beta c alone (alpha 0): 2e-3 * 0.75 + ulp(0.25) = 2^(-2-10)
    (torch.float16, 0.0, 100.0, 0.75, 0.25, 0.0015 + 2.0 ** -12),
]

# (activation, Lipschitz constant): fp16, alpha 1, T 10, |beta c| + |bias| 0.5, D_ref 1
_FUSED_CASES = [(None, 1.0), ("relu", 1.0), ("gelu", 1.13)]


def _pin_bound(m):
    for dt, alpha, T, cabs, dref, want in _BOUND_CASES:
        got = m.bound(np.array([T]), np.array([cabs]), np.array([dref]), alpha, dt)[0]
        assert abs(got - want) <= 1e-15 * max(want, 1e-300) or got == want, (dt, alpha, T, cabs, dref, got, want)
        # check() accepts just inside the hand budget and refuses just outside
        for side, ok in ((0.999, True), (1.001, False)):
            r = m.check(np.array([dref + side * want]), np.array([dref]), np.array([T]), np.array([cabs]),
                        alpha, dt)
            assert r.ok == ok, (dt, alpha, T, cabs, dref, side)


def _pin_check_fused(m):
    for act, lip in _FUSED_CASES:
        want = lip * 2e-3 * (10.0 + 0.5) + 2.0 ** -10
        for side, ok in ((0.999, True), (1.001, False)):
            r = m.check_fused(np.array([1.0 + side * want]), np.array([1.0]), np.array([10.0]), np.array([0.5]),
                              1.0, torch.float16, act)
            assert r.ok == ok, (act, side, want)
    # alpha enters by magnitude here too
    want = 2e-3 * (2.0 * 10.0 + 0.5) + 2.0 ** -10
    r = m.check_fused(np.array([1.0 + 1.001 * want]), np.array([1.0]), np.array([10.0]), np.array([0.5]),
                      -2.0, torch.float16, "relu")
    assert not r.ok
    r = m.check_fused(np.array([1.0 + 0.999 * want]), np.array([1.0]), np.array([10.0]), np.array([0.5]),
                      -2.0, torch.float16, "relu")
    assert r.ok


def test_bound_equals_hand_computed_budgets():
    _pin_bound(og)


def test_check_fused_equals_hand_computed_budgets():
    _pin_check_fused(og)


_BOUND_MUTANTS = {
    "coefficient_2e-2": ("return 2e-3 * (abs(alpha) * T + Cabs)", "return 2e-2 * (abs(alpha) * T + Cabs)"),
    "alpha_not_abs": ("return 2e-3 * (abs(alpha) * T + Cabs)", "return 2e-3 * (alpha * T + Cabs)"),
    "beta_c_dropped": ("return 2e-3 * (abs(alpha) * T + Cabs)", "return 2e-3 * (abs(alpha) * T)"),
    "ulp_dropped": ("+ Cabs) + ulp_out(Dref, dtype)", "+ Cabs)"),
    "fused_lipschitz_dropped": ("b = LIPSCHITZ[act] * 2e-3", "b = 2e-3"),
    "fused_coefficient": ("b = LIPSCHITZ[act] * 2e-3", "b = LIPSCHITZ[act] * 2e-2"),
    "fused_alpha_not_abs": ("(abs(alpha) * T.reshape(-1) + mag)", "(alpha * T.reshape(-1) + mag)"),
    "fused_mag_dropped": ("(abs(alpha) * T.reshape(-1) + mag)", "(abs(alpha) * T.reshape(-1))"),
    "fused_ulp_dropped": ("+ mag) + ulp_out(Dref, dtype)", "+ mag)"),
}


@pytest.mark.parametrize("name", sorted(_BOUND_MUTANTS))
def test_bound_mutant_is_caught(name, tmp_path):
    import importlib.util
    src = open(og.__file__).read()
    old, new = _BOUND_MUTANTS[name]
    assert src.count(old) == 1, name
    path = tmp_path / "gemm_mutant.py"
    path.write_text(src.replace(old, new))
    import sys
    modname = f"oracle_gemm_mutant_{name}"
    spec = importlib.util.spec_from_file_location(modname, path)
    mutant = importlib.util.module_from_spec(spec)
    sys.modules[modname] = mutant   # (its dataclasses look their module up there)
    try:
        spec.loader.exec_module(mutant)
    finally:
        sys.modules.pop(modname, None)
    caught = 0
    for pin in (_pin_bound, _pin_check_fused):
        try:
            pin(mutant)
        except AssertionError:
            caught += 1
    assert caught > 0, name
