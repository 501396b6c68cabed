"""Build the C-ABI shared library ``liblt.so`` in-tree with hipcc for gfx950.

    python -m layout_algebra_tiled_amd.build          # compile (always)

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled in device code; the objects go to ``_build/`` at the repo
root and the library next to this file, where the Python binding loads it.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "liblt.so")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["layout.cpp", "gemm.cpp", "device.hip", "gemm_kernels.hip"]
# The tiled kernel is compiled once per (dtype, A K-major?, B K-major?): each
# object holds one variant's kernels, and the objects build in parallel.
TILED_VARIANTS = [(dt, ak, bk) for dt in (1, 2) for ak in (1, 0) for bk in (1, 0)]

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", f"-I{INCLUDE}", f"-I{CSRC}",
          "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
          # device code: no packed fp32 instructions
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(job) -> str:
    src, defines, stem = job
    obj = os.path.join(BUILD, stem + ".o")
    cmd = [HIPCC, *COMMON, *defines, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if msgs.strip():
        sys.stderr.write(msgs + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = [("gemm_tiled.hip", [f"-DLT_TILED_DT={dt}", f"-DLT_TILED_AK={ak}", f"-DLT_TILED_BK={bk}"],
             f"gemm_tiled_{dt}{ak}{bk}") for dt, ak, bk in TILED_VARIANTS]
    jobs += [(src, [], os.path.splitext(src)[0]) for src in SOURCES]
    workers = min(len(jobs), max(1, min(16, os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(_compile, jobs))
    tmp = OUT + f".tmp{os.getpid()}"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build()
