"""ctypes declarations of the C ABI in include/lt.h (argument marshalling only).

The shared library is built in-tree by ``layout_algebra_tiled_amd.build``.
Loading fails loudly if it has not been built: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

LT_MAX_LEAVES = 32
LT_MAX_NODES = 64
LT_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024 + 4096

LT_OK = 0
STATUS_NAMES = {
    0: "LT_OK", 1: "LT_ERR_INVALID_ARGUMENT", 2: "LT_ERR_INVALID_LAYOUT", 3: "LT_ERR_NOT_ADMISSIBLE",
    4: "LT_ERR_NOT_DIVISIBLE", 5: "LT_ERR_OUT_OF_RANGE", 6: "LT_ERR_MISALIGNED_OPERAND",
    7: "LT_ERR_UNSUPPORTED", 8: "LT_ERR_ARCH_MISMATCH", 9: "LT_ERR_LDS_OVERFLOW", 10: "LT_ERR_WORKSPACE",
    11: "LT_ERR_HIP", 12: "LT_ERR_CAPACITY",
}
STATUS = {v: k for k, v in STATUS_NAMES.items()}

LT_F16, LT_BF16 = 1, 2
LT_KERNEL_AUTO, LT_KERNEL_WAVE16, LT_KERNEL_TILED, LT_KERNEL_SKINNY = 0, 1, 2, 3


class lt_layout(ctypes.Structure):
    _fields_ = [("nleaves", ctypes.c_int32), ("nnodes", ctypes.c_int32),
                ("shape", ctypes.c_int64 * LT_MAX_LEAVES), ("stride", ctypes.c_int64 * LT_MAX_LEAVES),
                ("tree", ctypes.c_int8 * LT_MAX_NODES)]


class lt_tensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("layout", lt_layout)]


class lt_gemm_options(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("split_k", ctypes.c_int32), ("persistent", ctypes.c_int32), ("tile_order", ctypes.c_int32)]


class lt_epilogue(ctypes.Structure):
    _fields_ = [("bias", ctypes.c_void_p), ("bias_stride", ctypes.c_int64), ("bias_per_row", ctypes.c_int32),
                ("activation", ctypes.c_int32), ("amax", ctypes.c_void_p)]


LT_ACT_NONE, LT_ACT_RELU, LT_ACT_GELU = 0, 1, 2


class lt_gemm_plan_info(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("tile_k", ctypes.c_int32), ("wave_m", ctypes.c_int32), ("wave_n", ctypes.c_int32),
                ("waves", ctypes.c_int32), ("stages", ctypes.c_int32), ("split_k", ctypes.c_int32),
                ("a_kmajor", ctypes.c_int32), ("b_kmajor", ctypes.c_int32), ("d_nmajor", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("lds_bytes", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("mfma_per_wave_kstep", ctypes.c_int64), ("mfma_m", ctypes.c_int32), ("mfma_n", ctypes.c_int32),
                ("mfma_k", ctypes.c_int32), ("sk_tiles", ctypes.c_int64), ("sk_workgroups", ctypes.c_int32),
                ("tiles", ctypes.c_int64), ("persistent", ctypes.c_int32), ("tile_order", ctypes.c_int32)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


_P = ctypes.POINTER
_L = _P(lt_layout)
_T = _P(lt_tensor)
_i32, _i64, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_vp = ctypes.c_void_p

# name: (argtypes, restype) — every function declared in include/lt.h
SIGNATURES = {
    "lt_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "lt_layout_validate": ([_L], ctypes.c_int),
    "lt_layout_parse": ([ctypes.c_char_p, _L], ctypes.c_int),
    "lt_layout_format": ([_L, ctypes.c_char_p, _sz, _P(_sz)], ctypes.c_int),
    "lt_make_layout": ([_i32, _P(_i64), _P(_i64), _L], ctypes.c_int),
    "lt_make_colmajor": ([_i32, _P(_i64), _L], ctypes.c_int),
    "lt_make_rowmajor": ([_i32, _P(_i64), _L], ctypes.c_int),
    "lt_make_tuple": ([_i32, _L, _L], ctypes.c_int),
    "lt_mode": ([_L, _i32, _L], ctypes.c_int),
    "lt_size": ([_L, _P(_i64)], ctypes.c_int),
    "lt_cosize": ([_L, _P(_i64)], ctypes.c_int),
    "lt_rank": ([_L, _P(_i32)], ctypes.c_int),
    "lt_depth": ([_L, _P(_i32)], ctypes.c_int),
    "lt_eval_index": ([_L, _i64, _P(_i64)], ctypes.c_int),
    "lt_eval_coord": ([_L, _P(_i64), _i32, _P(_i64)], ctypes.c_int),
    "lt_coalesce": ([_L, _L], ctypes.c_int),
    "lt_compose": ([_L, _L, _L], ctypes.c_int),
    "lt_complement": ([_L, _i64, _L], ctypes.c_int),
    "lt_logical_divide": ([_L, _L, _L], ctypes.c_int),
    "lt_logical_product": ([_L, _L, _L], ctypes.c_int),
    "lt_make_tv_layout": ([_i32, _P(_i64), _P(_i64), _P(ctypes.c_uint8), _L], ctypes.c_int),
    "lt_logical_divide_shape": ([_L, _i32, _P(_i64), _L], ctypes.c_int),
    "lt_zipped_divide": ([_L, _i32, _P(_i64), _L], ctypes.c_int),
    "lt_local_tile": ([_L, _i32, _P(_i64), _P(_i64), _P(ctypes.c_uint8), _P(_i64), _L], ctypes.c_int),
    "lt_local_partition": ([_L, _L, _i64, _P(ctypes.c_uint8), _P(_i64), _L], ctypes.c_int),
    "lt_device_check": ([ctypes.c_char_p, _sz], ctypes.c_int),
    "lt_set_arch_override": ([ctypes.c_char_p], ctypes.c_int),
    "lt_layout_eval_device": ([_L, _vp, _i64, _vp], ctypes.c_int),
    "lt_gather_device": ([_L, _vp, _vp, _i32, _i64, _vp], ctypes.c_int),
    "lt_gemm_plan": ([_T, _T, _T, _T, _i32, _P(lt_gemm_options), _P(lt_gemm_plan_info)], ctypes.c_int),
    "lt_gemm_can_implement": ([_T, _T, _T, _T, _i32, _P(lt_gemm_options)], ctypes.c_int),
    "lt_gemm_workspace_size": ([_T, _T, _T, _T, _i32, _P(lt_gemm_options), _P(_sz)], ctypes.c_int),
    "lt_gemm_run": ([_T, _T, _T, _T, ctypes.c_float, ctypes.c_float, _P(lt_gemm_options), _vp, _sz, _vp],
                    ctypes.c_int),
    "lt_gemm_run_ex": ([_T, _T, _T, _T, ctypes.c_float, ctypes.c_float, _P(lt_gemm_options), _P(lt_epilogue),
                        _vp, _sz, _vp], ctypes.c_int),
    "lt_gemm_run_noalloc": ([_T, _T, _T, _T, ctypes.c_float, ctypes.c_float, _P(lt_gemm_options), _P(lt_epilogue),
                             _vp], ctypes.c_int),
    "lt_version": ([], ctypes.c_char_p),
}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblt.so")
_lib = None


class LtError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))
        msg = lib().lt_status_string(status).decode() if _lib is not None else ""
        super().__init__(f"{what}: {self.name} ({msg})" if what else f"{self.name} ({msg})")


def lib():
    """The loaded C-ABI library. Raises if it was never built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m layout_algebra_tiled_amd.build` "
                               "(or __graft_entry__.build()); there is no fallback implementation")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def check(status: int, what: str = ""):
    if status != LT_OK:
        raise LtError(status, what)
