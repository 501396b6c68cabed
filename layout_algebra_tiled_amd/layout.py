"""Python face of the host layout algebra: every operation is one call into
the C ABI (include/lt.h); this module only converts arguments and results."""

from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple, Union

from ._lib import LtError, check, lib, lt_layout

IntTuple = Union[int, tuple]


def _fmt(t: IntTuple) -> str:
    if isinstance(t, (tuple, list)):
        return "(" + ",".join(_fmt(x) for x in t) + ")"
    return str(int(t))


class Layout:
    """A Shape:Stride layout held as the C ABI's lt_layout value."""

    __slots__ = ("_c",)

    def __init__(self, c: lt_layout):
        self._c = c

    # -- construction ------------------------------------------------------
    @staticmethod
    def parse(text: str) -> "Layout":
        c = lt_layout()
        check(lib().lt_layout_parse(text.encode(), ctypes.byref(c)), f"parse {text!r}")
        return Layout(c)

    @staticmethod
    def of(shape: IntTuple, stride: IntTuple) -> "Layout":
        """From nested Python tuples, e.g. Layout.of(((2,2),3), ((24,2),8))."""
        return Layout.parse(_fmt(shape) + ":" + _fmt(stride))

    @staticmethod
    def make(shape: Sequence[int], stride: Sequence[int]) -> "Layout":
        n = len(shape)
        s = (ctypes.c_int64 * n)(*shape)
        d = (ctypes.c_int64 * n)(*stride)
        c = lt_layout()
        check(lib().lt_make_layout(n, s, d, ctypes.byref(c)), "make_layout")
        return Layout(c)

    @staticmethod
    def colmajor(shape: Sequence[int]) -> "Layout":
        c = lt_layout()
        check(lib().lt_make_colmajor(len(shape), (ctypes.c_int64 * len(shape))(*shape), ctypes.byref(c)))
        return Layout(c)

    @staticmethod
    def rowmajor(shape: Sequence[int]) -> "Layout":
        c = lt_layout()
        check(lib().lt_make_rowmajor(len(shape), (ctypes.c_int64 * len(shape))(*shape), ctypes.byref(c)))
        return Layout(c)

    @staticmethod
    def tuple_of(*modes: "Layout") -> "Layout":
        arr = (lt_layout * len(modes))(*[m._c for m in modes])
        c = lt_layout()
        check(lib().lt_make_tuple(len(modes), arr, ctypes.byref(c)), "make_tuple")
        return Layout(c)

    # -- views -------------------------------------------------------------
    @property
    def c(self) -> lt_layout:
        return self._c

    def __str__(self) -> str:
        need = ctypes.c_size_t(0)
        buf = ctypes.create_string_buffer(4096)
        check(lib().lt_layout_format(ctypes.byref(self._c), buf, 4096, ctypes.byref(need)), "format")
        return buf.value.decode()

    __repr__ = __str__

    def __eq__(self, other) -> bool:
        return isinstance(other, Layout) and str(self) == str(other)

    def __hash__(self):
        return hash(str(self))

    def _tree(self) -> Tuple[IntTuple, IntTuple]:
        c = self._c
        code = list(c.tree[: c.nnodes])
        leaves = [(c.shape[i], c.stride[i]) for i in range(c.nleaves)]
        pos = [0, 0]

        def go():
            k = code[pos[0]]
            pos[0] += 1
            if k == 0:
                s, d = leaves[pos[1]]
                pos[1] += 1
                return s, d
            kids = [go() for _ in range(k)]
            return tuple(x[0] for x in kids), tuple(x[1] for x in kids)

        return go()

    @property
    def shape(self) -> IntTuple:
        return self._tree()[0]

    @property
    def stride(self) -> IntTuple:
        return self._tree()[1]

    def size(self) -> int:
        v = ctypes.c_int64()
        check(lib().lt_size(ctypes.byref(self._c), ctypes.byref(v)))
        return v.value

    def cosize(self) -> int:
        v = ctypes.c_int64()
        check(lib().lt_cosize(ctypes.byref(self._c), ctypes.byref(v)))
        return v.value

    @property
    def rank(self) -> int:
        v = ctypes.c_int32()
        check(lib().lt_rank(ctypes.byref(self._c), ctypes.byref(v)))
        return v.value

    def depth(self) -> int:
        v = ctypes.c_int32()
        check(lib().lt_depth(ctypes.byref(self._c), ctypes.byref(v)))
        return v.value

    def mode(self, i: int) -> "Layout":
        c = lt_layout()
        check(lib().lt_mode(ctypes.byref(self._c), i, ctypes.byref(c)), f"mode {i}")
        return Layout(c)

    def __call__(self, x) -> int:
        v = ctypes.c_int64()
        if isinstance(x, int):
            check(lib().lt_eval_index(ctypes.byref(self._c), x, ctypes.byref(v)), f"eval {x}")
        else:
            n = len(x)
            arr = (ctypes.c_int64 * n)(*x)
            check(lib().lt_eval_coord(ctypes.byref(self._c), arr, n, ctypes.byref(v)), f"eval {x}")
        return v.value

    # -- algebra -------------------------------------------------------------
    def coalesce(self) -> "Layout":
        c = lt_layout()
        check(lib().lt_coalesce(ctypes.byref(self._c), ctypes.byref(c)), "coalesce")
        return Layout(c)

    def compose(self, B: "Layout") -> "Layout":
        c = lt_layout()
        check(lib().lt_compose(ctypes.byref(self._c), ctypes.byref(B._c), ctypes.byref(c)), "compose")
        return Layout(c)

    def complement(self, M: int) -> "Layout":
        c = lt_layout()
        check(lib().lt_complement(ctypes.byref(self._c), M, ctypes.byref(c)), "complement")
        return Layout(c)

    def logical_divide(self, tiler) -> "Layout":
        c = lt_layout()
        if isinstance(tiler, int):
            tiler = Layout.make([tiler], [1])
        if isinstance(tiler, Layout):
            check(lib().lt_logical_divide(ctypes.byref(self._c), ctypes.byref(tiler._c), ctypes.byref(c)),
                  "logical_divide")
        else:
            t = tuple(tiler)
            arr = (ctypes.c_int64 * len(t))(*t)
            check(lib().lt_logical_divide_shape(ctypes.byref(self._c), len(t), arr, ctypes.byref(c)),
                  "logical_divide")
        return Layout(c)

    def logical_product(self, B: "Layout") -> "Layout":
        c = lt_layout()
        check(lib().lt_logical_product(ctypes.byref(self._c), ctypes.byref(B._c), ctypes.byref(c)),
              "logical_product")
        return Layout(c)

    @staticmethod
    def tv(thr: Sequence[int], val: Sequence[int], blocked: Optional[Sequence[int]] = None) -> "Layout":
        """Thread-value layout of a column-major tile of extents thr[i]*val[i]
        (lt_make_tv_layout): ((threads), (values)) -> offset."""
        n = len(thr)
        t = (ctypes.c_int64 * n)(*thr)
        v = (ctypes.c_int64 * n)(*val)
        b = (ctypes.c_uint8 * n)(*blocked) if blocked is not None else None
        c = lt_layout()
        check(lib().lt_make_tv_layout(n, t, v, b, ctypes.byref(c)), "make_tv_layout")
        return Layout(c)

    def zipped_divide(self, tiler: Sequence[int]) -> "Layout":
        t = tuple(tiler)
        arr = (ctypes.c_int64 * len(t))(*t)
        c = lt_layout()
        check(lib().lt_zipped_divide(ctypes.byref(self._c), len(t), arr, ctypes.byref(c)), "zipped_divide")
        return Layout(c)

    def local_tile(self, tiler: Sequence[int], coord: Sequence[Optional[int]],
                   step: Optional[Sequence[int]] = None) -> Tuple[int, "Layout"]:
        n = len(tiler)
        t = (ctypes.c_int64 * n)(*tiler)
        cd = (ctypes.c_int64 * n)(*[-1 if x is None else x for x in coord])
        st = (ctypes.c_uint8 * n)(*step) if step is not None else None
        off = ctypes.c_int64()
        c = lt_layout()
        check(lib().lt_local_tile(ctypes.byref(self._c), n, t, cd, st, ctypes.byref(off), ctypes.byref(c)),
              "local_tile")
        return off.value, Layout(c)

    def local_partition(self, thr: "Layout", t: int, step: Optional[Sequence[int]] = None) -> Tuple[int, "Layout"]:
        st = (ctypes.c_uint8 * len(step))(*step) if step is not None else None
        off = ctypes.c_int64()
        c = lt_layout()
        check(lib().lt_local_partition(ctypes.byref(self._c), ctypes.byref(thr._c), t, st, ctypes.byref(off),
                                       ctypes.byref(c)), "local_partition")
        return off.value, Layout(c)


__all__ = ["Layout", "LtError"]
