"""GEMM and device layout maps on torch-allocated device memory.

Marshalling only: tensors are turned into (pointer, dtype, layout) and handed
to the C ABI; every step of the computation runs in the library's kernels.
PyTorch provides device memory and the current stream.
"""

from __future__ import annotations

import ctypes
from typing import Optional, Union

import torch

from . import _lib as L
from .layout import Layout

_DT = {torch.float16: L.LT_F16, torch.bfloat16: L.LT_BF16}
KERNELS = {"auto": L.LT_KERNEL_AUTO, "wave16": L.LT_KERNEL_WAVE16, "tiled": L.LT_KERNEL_TILED,
           "skinny": L.LT_KERNEL_SKINNY}
KERNEL_NAMES = {v: k for k, v in KERNELS.items()}


def tensor_desc(t: torch.Tensor, layout: Optional[Layout] = None) -> L.lt_tensor:
    """(pointer, dtype, layout) of a tensor; the layout defaults to the view's
    own shape and strides. With an explicit layout, ``t`` is the storage and
    the layout addresses it from ``t.data_ptr()``: its cosize (the elements it
    reaches) must fit in what the storage holds from there, else ValueError
    (the C ABI sees only a pointer and cannot check this)."""
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if layout is None:
        layout = Layout.make(list(t.shape), list(t.stride()))
    else:
        room = t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()
        if layout.size() > 0 and layout.cosize() > room:
            raise ValueError(f"layout {layout} reaches {layout.cosize()} elements; the storage holds {room} "
                             f"from the tensor's first element")
    d = L.lt_tensor()
    d.ptr = t.data_ptr()
    d.dtype = _DT[t.dtype]
    d.layout = layout.c
    return d


TILE_ORDERS = {None: 0, "raster": 1, "superblock": 2, "raster_krev": 3}


def _opts(kernel: Union[str, int], tile=None, split_k: int = 0, persistent=None,
          tile_order=None) -> L.lt_gemm_options:
    o = L.lt_gemm_options()
    o.kernel = KERNELS[kernel] if isinstance(kernel, str) else int(kernel)
    o.tile_m, o.tile_n = tile if tile else (0, 0)
    o.split_k = split_k
    o.persistent = 0 if persistent is None else (2 if persistent else 1)
    if tile_order not in TILE_ORDERS:
        raise ValueError(f"unknown tile order {tile_order!r}")
    o.tile_order = TILE_ORDERS[tile_order]
    return o


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def plan(A, B, D, C=None, beta: float = 0.0, kernel="auto", tile=None, split_k=0, layouts=None,
         persistent=None, tile_order=None) -> dict:
    la = layouts or {}
    dA, dB, dD = tensor_desc(A, la.get("A")), tensor_desc(B, la.get("B")), tensor_desc(D, la.get("D"))
    dC = tensor_desc(C, la.get("C")) if C is not None else None
    info = L.lt_gemm_plan_info()
    o = _opts(kernel, tile, split_k, persistent, tile_order)
    L.check(L.lib().lt_gemm_plan(ctypes.byref(dA), ctypes.byref(dB), ctypes.byref(dC) if dC else None,
                                 ctypes.byref(dD), int(beta != 0.0), ctypes.byref(o), ctypes.byref(info)),
            "gemm_plan")
    r = info.as_dict()
    r["kernel_name"] = KERNEL_NAMES.get(r["kernel"], "?")
    return r


ACTIVATIONS = {None: L.LT_ACT_NONE, "none": L.LT_ACT_NONE, "relu": L.LT_ACT_RELU, "gelu": L.LT_ACT_GELU}


def _epilogue(bias, bias_stride, bias_per_row, activation, amax) -> Optional[L.lt_epilogue]:
    """The fused-epilogue descriptor, or None for the plain alpha/beta one."""
    if bias is None and activation in (None, "none") and amax is None:
        return None
    if activation not in ACTIVATIONS:
        raise ValueError(f"unknown activation {activation!r}")
    if amax is not None and amax.dtype != torch.float32:
        raise ValueError("amax must be a float32 device tensor")
    return L.lt_epilogue(bias.data_ptr() if bias is not None else None, int(bias_stride), int(bool(bias_per_row)),
                         ACTIVATIONS[activation], amax.data_ptr() if amax is not None else None)


def gemm(A: torch.Tensor, B: torch.Tensor, D: torch.Tensor, C: Optional[torch.Tensor] = None,
         alpha: float = 1.0, beta: float = 0.0, *, kernel="auto", tile=None, split_k: int = 0,
         persistent: Optional[bool] = None, tile_order: Optional[str] = None, layouts: Optional[dict] = None,
         workspace: Optional[torch.Tensor] = None, stream=None,
         bias: Optional[torch.Tensor] = None, bias_stride: int = 1, bias_per_row: bool = False,
         activation: Optional[str] = None, amax: Optional[torch.Tensor] = None) -> None:
    """D = act(alpha * A @ B + beta * C + bias) (asynchronous on ``stream``).
    ``bias`` (D's dtype, one value per column, or per row with
    ``bias_per_row``), ``activation`` ("relu", "gelu") and ``amax`` (a float32
    device scalar receiving max |D|) select the fused epilogue. ``persistent``
    (None: the planner's choice) forces the persistent launch on or off;
    ``tile_order`` ("raster", "superblock", "raster_krev"; None: the
    planner's choice) sets the order of the data-parallel launch's tiles."""
    la = layouts or {}
    dA, dB, dD = tensor_desc(A, la.get("A")), tensor_desc(B, la.get("B")), tensor_desc(D, la.get("D"))
    dC = tensor_desc(C, la.get("C")) if C is not None else None
    o = _opts(kernel, tile, split_k, persistent, tile_order)
    ws_ptr, ws_bytes = None, 0
    sid = _stream(stream)
    if workspace is None:
        # Size it (the library refuses a run whose workspace is too small,
        # so a caller-provided one needs no query). The tensor is freed when
        # this call returns while the kernels may still be using it on the
        # launch stream: record that stream so the caching allocator does
        # not hand the memory out before they finish.
        need = ctypes.c_size_t(0)
        L.check(L.lib().lt_gemm_workspace_size(ctypes.byref(dA), ctypes.byref(dB),
                                               ctypes.byref(dC) if dC else None, ctypes.byref(dD),
                                               int(beta != 0.0), ctypes.byref(o), ctypes.byref(need)),
                "gemm_workspace_size")
        if need.value:
            workspace = torch.empty(need.value, dtype=torch.uint8, device=D.device)
            workspace.record_stream(torch.cuda.ExternalStream(sid, device=D.device))
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    epi = _epilogue(bias, bias_stride, bias_per_row, activation, amax)
    L.check(L.lib().lt_gemm_run_ex(ctypes.byref(dA), ctypes.byref(dB), ctypes.byref(dC) if dC else None,
                                   ctypes.byref(dD), float(alpha), float(beta), ctypes.byref(o),
                                   ctypes.byref(epi) if epi is not None else None, ws_ptr, ws_bytes,
                                   sid), "gemm_run")


def gemm_noalloc(A: torch.Tensor, B: torch.Tensor, D: torch.Tensor, C: Optional[torch.Tensor] = None,
                 alpha: float = 1.0, beta: float = 0.0, *, kernel="auto", tile=None, split_k: int = 0,
                 persistent: Optional[bool] = None, tile_order: Optional[str] = None,
                 layouts: Optional[dict] = None, stream=None,
                 bias: Optional[torch.Tensor] = None,
                 bias_stride: int = 1, bias_per_row: bool = False, activation: Optional[str] = None,
                 amax: Optional[torch.Tensor] = None) -> None:
    """gemm() through lt_gemm_run_noalloc: no workspace, no device memory
    allocated; the scratch comes from the library's static per-GPU array
    (calls that overlap on one GPU race on it)."""
    la = layouts or {}
    dA, dB, dD = tensor_desc(A, la.get("A")), tensor_desc(B, la.get("B")), tensor_desc(D, la.get("D"))
    dC = tensor_desc(C, la.get("C")) if C is not None else None
    o = _opts(kernel, tile, split_k, persistent, tile_order)
    epi = _epilogue(bias, bias_stride, bias_per_row, activation, amax)
    L.check(L.lib().lt_gemm_run_noalloc(ctypes.byref(dA), ctypes.byref(dB), ctypes.byref(dC) if dC else None,
                                        ctypes.byref(dD), float(alpha), float(beta), ctypes.byref(o),
                                        ctypes.byref(epi) if epi is not None else None, _stream(stream)),
            "gemm_run_noalloc")


def layout_eval_device(layout: Layout, out: torch.Tensor, n: Optional[int] = None, stream=None) -> None:
    """out[x] = layout(x) for x < n (int64 device tensor)."""
    assert out.dtype == torch.int64 and out.is_contiguous()
    n = out.numel() if n is None else n
    L.check(L.lib().lt_layout_eval_device(ctypes.byref(layout.c), out.data_ptr(), n, _stream(stream)),
            "layout_eval_device")


def gather_device(layout: Layout, src: torch.Tensor, dst: torch.Tensor, n: Optional[int] = None,
                  stream=None) -> None:
    """dst[x] = src[layout(x)] for x < n."""
    assert src.dtype == dst.dtype and dst.is_contiguous()
    n = dst.numel() if n is None else n
    L.check(L.lib().lt_gather_device(ctypes.byref(layout.c), src.data_ptr(), dst.data_ptr(), src.element_size(),
                                     n, _stream(stream)), "gather_device")


def device_check() -> str:
    buf = ctypes.create_string_buffer(64)
    L.check(L.lib().lt_device_check(buf, 64), "device_check")
    return buf.value.decode()
