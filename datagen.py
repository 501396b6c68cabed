"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no GEMM or layout-algebra arithmetic: it draws numbers,
rounds them once to the operand dtype and places them in memory in the
requested major order. Both the oracle side and the GPU side are fed from it.

Recipe (the pages use no dataset; these are the five synthetic workloads the
build is measured on):

* RNG: ``numpy.random.default_rng(seed)`` with seed = 1000*cfg + {A: 0, B: 1,
  C: 2}. Values are drawn in float64 in logical row-major (i, j) order and then
  rounded once to fp16/bf16 with round-to-nearest-even (torch CPU ``.to``).
* Distributions: uniform[-1, 1]; N(0,1)/sqrt(K) (both operands of the 8192^3
  case); N(0,1) activations and N(0, sigma=0.02) weights (skinny case).
* Memory: an operand is a flat storage plus a rank-2 Shape:Stride view in
  elements. "row" major stores (rows, ld) with stride (ld, 1); "col" major
  stores (cols, ld) with stride (1, ld). Padding elements beyond the logical
  extent (ld > extent) hold NaN so that a kernel reading them is caught.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np
import torch


@dataclass
class Matrix:
    store: torch.Tensor            # 1-D CPU tensor
    shape: Tuple[int, int]
    stride: Tuple[int, int]

    @property
    def dtype(self):
        return self.store.dtype

    def view(self) -> torch.Tensor:
        return torch.as_strided(self.store, self.shape, self.stride)

    def to(self, device) -> "Matrix":
        return Matrix(self.store.to(device), self.shape, self.stride)


def draw(rows: int, cols: int, dist: str, seed: int, k_for_scale: int = 1) -> np.ndarray:
    rng = np.random.default_rng(seed)
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, size=(rows, cols))
    if dist == "normal_over_sqrtk":
        return rng.standard_normal(size=(rows, cols)) / np.sqrt(float(k_for_scale))
    if dist == "normal":
        return rng.standard_normal(size=(rows, cols))
    if dist == "normal_0.02":
        return rng.standard_normal(size=(rows, cols)) * 0.02
    if dist == "smallint":
        return rng.integers(-2, 3, size=(rows, cols)).astype(np.float64)
    raise ValueError(dist)


def place(values: np.ndarray, dtype: torch.dtype, major: str, ld: Optional[int] = None) -> Matrix:
    """Round once to ``dtype`` and store in ``major`` order with leading
    dimension ``ld`` (default: tight)."""
    rows, cols = values.shape
    t = torch.from_numpy(np.ascontiguousarray(values)).to(dtype)
    if major == "row":
        ld = cols if ld is None else ld
        assert ld >= cols
        buf = torch.full((max(rows, 1), ld), float("nan"), dtype=dtype)
        buf[:rows, :cols] = t
        return Matrix(buf.reshape(-1)[: max(rows * ld, 1)].clone(), (rows, cols), (ld, 1))
    if major == "col":
        ld = rows if ld is None else ld
        assert ld >= rows
        buf = torch.full((max(cols, 1), ld), float("nan"), dtype=dtype)
        buf[:cols, :rows] = t.t()
        return Matrix(buf.reshape(-1)[: max(cols * ld, 1)].clone(), (rows, cols), (1, ld))
    raise ValueError(major)


def matrix(rows: int, cols: int, dtype: torch.dtype, major: str, dist: str, seed: int,
           ld: Optional[int] = None, k_for_scale: int = 1) -> Matrix:
    return place(draw(rows, cols, dist, seed, k_for_scale), dtype, major, ld)


def zeros(rows: int, cols: int, dtype: torch.dtype, major: str = "row", ld: Optional[int] = None) -> Matrix:
    return place(np.zeros((rows, cols)), dtype, major, ld)


@dataclass
class GemmCase:
    """One synthetic GEMM workload: D = alpha*A*B + beta*C."""
    cfg: int
    name: str
    dtype: torch.dtype
    M: int
    N: int
    K: int
    a_major: str                   # "row" = K-major A, "col" = M-major A
    b_major: str                   # "col" = K-major B, "row" = N-major B
    c_major: str
    alpha: float
    beta: float
    dist_a: str
    dist_b: str
    dist_c: str = "uniform"
    tile: Optional[Tuple[int, int]] = None      # explicit block tile, if the workload fixes one
    extra: dict = field(default_factory=dict)

    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def bytes(self) -> int:
        """Algorithmic bytes: A and B read once, C read if beta != 0, D written once."""
        e = torch.finfo(self.dtype).bits // 8
        n = self.M * self.K + self.K * self.N + self.M * self.N
        if self.beta != 0.0:
            n += self.M * self.N
        return n * e

    def make(self, seed_base: Optional[int] = None):
        """(A, B, C, D) CPU matrices; D is zero-filled in C's major order."""
        s = 1000 * self.cfg if seed_base is None else seed_base
        A = matrix(self.M, self.K, self.dtype, self.a_major, self.dist_a, s + 0, k_for_scale=self.K)
        B = matrix(self.K, self.N, self.dtype, self.b_major, self.dist_b, s + 1, k_for_scale=self.K)
        if self.beta != 0.0:
            C = matrix(self.M, self.N, self.dtype, self.c_major, self.dist_c, s + 2)
        else:
            C = zeros(self.M, self.N, self.dtype, self.c_major)
        D = zeros(self.M, self.N, self.dtype, self.c_major)
        return A, B, C, D


CONFIGS = {
    1: GemmCase(1, "fp16 256x128x64, 16x16 tiles by zipped_divide", torch.float16,
                256, 128, 64, "row", "col", "row", 1.0, 0.0, "uniform", "uniform", tile=(16, 16)),
    2: GemmCase(2, "fp16 4096^3, K-major A and B, beta=0.5", torch.float16,
                4096, 4096, 4096, "row", "col", "row", 1.0, 0.5, "uniform", "uniform", "uniform"),
    3: GemmCase(3, "bf16 8192^3, K-major A and B", torch.bfloat16,
                8192, 8192, 8192, "row", "col", "row", 1.0, 0.0,
                "normal_over_sqrtk", "normal_over_sqrtk"),
    4: GemmCase(4, "fp16 6144x4096x2048, M-major A, N-major B, alpha=2, beta=-1", torch.float16,
                6144, 4096, 2048, "col", "row", "row", 2.0, -1.0, "uniform", "uniform", "uniform"),
    5: GemmCase(5, "bf16 skinny 32x8192x8192, K-major B", torch.bfloat16,
                32, 8192, 8192, "row", "col", "row", 1.0, 0.0, "normal", "normal_0.02"),
}


def config(n: int) -> GemmCase:
    return CONFIGS[n]
