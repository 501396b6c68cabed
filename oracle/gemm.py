"""Reference (oracle) GEMM wrapper and the error-bound check.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product never does.

The arithmetic lives in ``gemm_oracle.c`` (plain fp64 i-j-k loops, compiled
with gcc -O2 -fopenmp and no fast-math). This file only widens 16-bit inputs
to float64 (exact), calls the C loops, and evaluates the per-element bound

    |D - D_ref| <= 2e-3 * (|alpha| * sum_k |a_ik b_kj| + |beta c_ij|) + ulp_out(D_ref)

where ulp_out is the spacing of the output format at |D_ref| (READING: the
bound names "one output-format ulp" without defining it; this is the
spacing of consecutive representable values at that magnitude). The
style of the check — the CPU sums in double over the very same half values the
GPU read, and reports the worst element as a fraction of its budget — follows
"CUTLASS and CuTe layouts", "Two programs: the algebra, then the GEMM" and
"Results".
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_gemm.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle (gcc, -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
                               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        d, i64 = ctypes.POINTER(ctypes.c_double), ctypes.c_int64
        lib.oracle_gemm_points.argtypes = [d, i64, i64, d, i64, i64, i64,
                                           ctypes.POINTER(i64), i64, d, d]
        lib.oracle_gemm_rows.argtypes = [d, i64, i64, d, i64, i64, i64, i64,
                                         ctypes.POINTER(i64), i64, d, d]
        lib.oracle_epilogue_points.argtypes = [d, d, i64, i64, ctypes.POINTER(i64), i64,
                                               ctypes.c_double, ctypes.c_double, d, d]
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


@dataclass
class Operand:
    """A rank-2 operand: flat storage plus a Shape:Stride layout in elements."""
    store: torch.Tensor          # 1-D CPU tensor (fp16, bf16, fp32 or fp64)
    shape: Tuple[int, int]
    stride: Tuple[int, int]

    def widened(self) -> np.ndarray:
        """Exact widening of the 16-bit values to float64."""
        t = self.store.detach().to("cpu").reshape(-1)
        return np.ascontiguousarray(t.to(torch.float64).numpy())


def _dp(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _ip(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def gemm_points(A: Operand, B: Operand, ij: np.ndarray,
                Aw: Optional[np.ndarray] = None, Bw: Optional[np.ndarray] = None):
    """S_ij = sum_k a_ik b_kj and T_ij = sum_k |a_ik b_kj| at the given (i, j)."""
    lib = _load()
    M, K = A.shape
    K2, N = B.shape
    assert K == K2, "inner dimensions differ"
    ij = np.ascontiguousarray(np.asarray(ij, dtype=np.int64).reshape(-1, 2))
    assert ij.size == 0 or (ij[:, 0].max() < M and ij[:, 1].max() < N and ij.min() >= 0)
    Aw = A.widened() if Aw is None else Aw
    Bw = B.widened() if Bw is None else Bw
    S = np.zeros(len(ij), dtype=np.float64)
    T = np.zeros(len(ij), dtype=np.float64)
    lib.oracle_gemm_points(_dp(Aw), A.stride[0], A.stride[1], _dp(Bw), B.stride[0], B.stride[1],
                           K, _ip(ij), len(ij), _dp(S), _dp(T))
    return S, T


def gemm_rows(A: Operand, B: Operand, rows: Sequence[int],
              Aw: Optional[np.ndarray] = None, Bw: Optional[np.ndarray] = None):
    """S and T for whole output rows (row-major len(rows) x N arrays)."""
    lib = _load()
    M, K = A.shape
    _, N = B.shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    Aw = A.widened() if Aw is None else Aw
    Bw = B.widened() if Bw is None else Bw
    S = np.zeros((len(rows), N), dtype=np.float64)
    T = np.zeros((len(rows), N), dtype=np.float64)
    lib.oracle_gemm_rows(_dp(Aw), A.stride[0], A.stride[1], _dp(Bw), B.stride[0], B.stride[1],
                         N, K, _ip(rows), len(rows), _dp(S), _dp(T))
    return S, T


def epilogue(S: np.ndarray, C: Optional[Operand], ij: np.ndarray, alpha: float, beta: float):
    """D_ref = alpha*S + beta*c and |beta*c| at the points (C unread if beta == 0)."""
    lib = _load()
    ij = np.ascontiguousarray(np.asarray(ij, dtype=np.int64).reshape(-1, 2))
    S = np.ascontiguousarray(S.reshape(-1), dtype=np.float64)
    Dref = np.zeros(len(ij), dtype=np.float64)
    Cabs = np.zeros(len(ij), dtype=np.float64)
    if beta != 0.0:
        assert C is not None
        Cw, sc0, sc1 = C.widened(), C.stride[0], C.stride[1]
    else:
        Cw, sc0, sc1 = np.zeros(1), 0, 0
    lib.oracle_epilogue_points(_dp(S), _dp(Cw), sc0, sc1, _ip(ij), len(ij),
                               float(alpha), float(beta), _dp(Dref), _dp(Cabs))
    return Dref, Cabs


# ---------------------------------------------------------------------------
# The bound
# ---------------------------------------------------------------------------

_FMT = {
    # dtype: (mantissa bits after the point, minimum normal exponent)
    torch.float16: (10, -14),
    torch.bfloat16: (7, -126),
}


def ulp_out(x: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """Spacing of the output format at |x|: 2**(max(floor(log2|x|), emin) - p);
    at x == 0 the smallest subnormal 2**(emin - p)."""
    p, emin = _FMT[dtype]
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(x)          # x = m * 2**e, m in [0.5, 1)  =>  floor(log2 x) = e - 1
    e = np.where(x == 0, emin, np.maximum(e - 1, emin))
    return np.ldexp(1.0, (e - p).astype(np.int64))


def bound(T: np.ndarray, Cabs: np.ndarray, Dref: np.ndarray, alpha: float,
          dtype: torch.dtype) -> np.ndarray:
    return 2e-3 * (abs(alpha) * T + Cabs) + ulp_out(Dref, dtype)


@dataclass
class CheckResult:
    ok: bool
    n: int
    n_bad: int
    worst_fraction: float       # max |err| / bound ("fraction of budget")
    worst_index: int
    nonfinite: int

    def __str__(self):
        return (f"{self.n - self.n_bad}/{self.n} within bound, worst {self.worst_fraction:.4f} "
                f"of budget (point {self.worst_index}), non-finite {self.nonfinite}")


def check(D: np.ndarray, Dref: np.ndarray, T: np.ndarray, Cabs: np.ndarray,
          alpha: float, dtype: torch.dtype) -> CheckResult:
    D = np.asarray(D, dtype=np.float64).reshape(-1)
    Dref = Dref.reshape(-1)
    b = bound(T.reshape(-1), Cabs.reshape(-1), Dref, alpha, dtype)
    finite = np.isfinite(D)
    err = np.where(finite, np.abs(D - Dref), np.inf)
    frac = err / b
    bad = ~(err <= b)
    wi = int(np.argmax(frac)) if len(frac) else -1
    return CheckResult(ok=not bad.any(), n=len(D), n_bad=int(bad.sum()),
                       worst_fraction=float(frac[wi]) if len(frac) else 0.0,
                       worst_index=wi, nonfinite=int((~finite).sum()))


def read_points(D: Operand, ij: np.ndarray) -> np.ndarray:
    """D(i, j) through D's layout, widened to float64."""
    Dw = D.widened()
    ij = np.asarray(ij, dtype=np.int64).reshape(-1, 2)
    return Dw[ij[:, 0] * D.stride[0] + ij[:, 1] * D.stride[1]]


# ---------------------------------------------------------------------------
# Fused epilogue: bias and activation ("CUTLASS, in depth", "Epilogue fusion")
# ---------------------------------------------------------------------------

def _erf(x: np.ndarray) -> np.ndarray:
    from scipy.special import erf   # a library primitive used as one step
    return erf(x)


def activation(x: np.ndarray, act: Optional[str]) -> np.ndarray:
    """READING: the page names ReLU-style activation and GELU without a
    formula. ReLU(x) = x if x > 0 else 0; GELU(x) = x * Phi(x), Phi the
    standard normal CDF, Phi(x) = (1 + erf(x / sqrt 2)) / 2 (exact, not the
    tanh approximation)."""
    x = np.asarray(x, dtype=np.float64)
    if act in (None, "none"):
        return x
    if act == "relu":
        return np.where(x > 0, x, 0.0)
    if act == "gelu":
        return x * 0.5 * (1.0 + _erf(x / np.sqrt(2.0)))
    raise ValueError(f"unknown activation {act!r}")


# |act(x) - act(y)| <= L |x - y|: ReLU 1; GELU's slope Phi(x) + x phi(x) peaks
# at x = sqrt 2, Phi(sqrt 2) + sqrt(2) phi(sqrt 2) = 1.1289..., bounded by 1.13.
LIPSCHITZ = {None: 1.0, "none": 1.0, "relu": 1.0, "gelu": 1.13}


def fused_epilogue(Dpre: np.ndarray, Cabs: np.ndarray, ij: np.ndarray, bias: Optional[torch.Tensor],
                   bias_stride: int, bias_per_row: bool, act: Optional[str]):
    """D_ref = act(alpha*S + beta*c + bias) from D_pre = alpha*S + beta*c at the
    points, and the magnitude |beta c| + |bias| that enters the bound."""
    ij = np.asarray(ij, dtype=np.int64).reshape(-1, 2)
    b = np.zeros(len(ij))
    if bias is not None:
        bw = bias.detach().to("cpu").reshape(-1).to(torch.float64).numpy()
        idx = ij[:, 0] if bias_per_row else ij[:, 1]
        b = bw[idx * bias_stride]
    x = Dpre.reshape(-1) + b
    return activation(x, act), Cabs.reshape(-1) + np.abs(b)


def check_fused(D: np.ndarray, Dref: np.ndarray, T: np.ndarray, mag: np.ndarray, alpha: float,
                dtype: torch.dtype, act: Optional[str]) -> CheckResult:
    """The GEMM bound carried through the activation's Lipschitz constant:
    |D - D_ref| <= L * 2e-3 * (|alpha| T + |beta c| + |bias|) + ulp_out(D_ref)."""
    D = np.asarray(D, dtype=np.float64).reshape(-1)
    Dref = Dref.reshape(-1)
    b = LIPSCHITZ[act] * 2e-3 * (abs(alpha) * T.reshape(-1) + mag) + ulp_out(Dref, dtype)
    finite = np.isfinite(D)
    err = np.where(finite, np.abs(D - Dref), np.inf)
    frac = err / b
    bad = ~(err <= b)
    wi = int(np.argmax(frac)) if len(frac) else -1
    return CheckResult(ok=not bad.any(), n=len(D), n_bad=int(bad.sum()),
                       worst_fraction=float(frac[wi]) if len(frac) else 0.0,
                       worst_index=wi, nonfinite=int((~finite).sum()))
