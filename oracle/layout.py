"""Reference (oracle) Shape:Stride layout algebra — plain, slow, CPU only.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module. The product path (the C-ABI library
and its Python binding) never imports, calls or links anything under
``oracle/``, and this module imports nothing from the product.

Sources, cited by page title and section (the pages are the authority on what
is computed):

* "CUTLASS and CuTe layouts" (Day 84), sections "A layout is a shape and a
  stride" and "Two programs: the algebra, then the GEMM".
* "3.5 CUTLASS II — CuTe 레이아웃·텐서", sections 3.5.3 to 3.5.7.
* "Layouts as Algebra: CUTLASS & CuTe", sections "The formula gets a name",
  "One notation, and no more transposes", "A shape is a tree", "Composition,
  worked by hand", "Divide is tiling", "The threads are a layout too" and
  "The kernel, in three lines".

A layout is a pair of congruent nested tuples ``(shape, stride)`` of
non-negative Python ints. Everything here is written for clarity: functions
are evaluated by enumeration wherever the definition is an enumeration.
Readings of points the pages leave open are marked READING.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, List, Sequence, Tuple, Union

IntTuple = Union[int, tuple]


class NotAdmissible(ValueError):
    """The requested composition/complement has no layout (pages: composition
    is not always defined; "Layouts as Algebra", "Composition, worked by hand")."""


class NotDivisible(ValueError):
    """A tiler does not divide the mode it tiles (3.5 CUTLASS II, 3.5.8/3.5.10)."""


# --------------------------------------------------------------------------
# Tuples
# --------------------------------------------------------------------------

def flatten(t: IntTuple) -> Tuple[int, ...]:
    """Leaves of a nested tuple, left to right."""
    if isinstance(t, tuple):
        out: List[int] = []
        for x in t:
            out.extend(flatten(x))
        return tuple(out)
    return (t,)


def congruent(a: IntTuple, b: IntTuple) -> bool:
    """Same tree: every extent has exactly one stride opposite it
    ("Layouts as Algebra", "A shape is a tree")."""
    if isinstance(a, tuple) != isinstance(b, tuple):
        return False
    if not isinstance(a, tuple):
        return True
    return len(a) == len(b) and all(congruent(x, y) for x, y in zip(a, b))


def product(t: IntTuple) -> int:
    p = 1
    for s in flatten(t):
        p *= s
    return p


def _rebuild(template: IntTuple, leaves: Sequence[int]) -> IntTuple:
    """Put ``leaves`` back into the tree of ``template``."""
    it = iter(leaves)

    def go(t):
        if isinstance(t, tuple):
            return tuple(go(x) for x in t)
        return next(it)

    return go(template)


# --------------------------------------------------------------------------
# The layout value and its evaluation
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Layout:
    shape: IntTuple
    stride: IntTuple

    def __post_init__(self):
        if not congruent(self.shape, self.stride):
            raise ValueError(f"shape {self.shape} and stride {self.stride} are not congruent")
        for s in flatten(self.shape):
            if not isinstance(s, int) or s < 0:
                raise ValueError(f"extent {s!r} must be an int >= 0")
        for d in flatten(self.stride):
            if not isinstance(d, int) or d < 0:
                raise ValueError(f"stride {d!r} must be an int >= 0 (READING: negatives rejected)")

    # -- queries ----------------------------------------------------------
    @property
    def rank(self) -> int:
        """Number of top-level modes (a bare integer shape is one mode)."""
        return len(self.shape) if isinstance(self.shape, tuple) else 1

    def mode(self, i: int) -> "Layout":
        if not isinstance(self.shape, tuple):
            if i != 0:
                raise IndexError(i)
            return self
        return Layout(self.shape[i], self.stride[i])

    def size(self) -> int:
        return size(self)

    def __call__(self, x) -> int:
        return evaluate(self, x)

    def __str__(self) -> str:
        return format_layout(self)


def size(L: Layout) -> int:
    """Number of coordinates: product of all extents (3.5 CUTLASS II, 3.5.5)."""
    return product(L.shape)


def unravel(shape: IntTuple, x: int) -> List[int]:
    """1-D index to natural (per-leaf) coordinate, first leaf fastest — the
    colexicographic order ("Layouts as Algebra", "The formula gets a name";
    3.5 CUTLASS II, 3.5.4)."""
    if not 0 <= x < product(shape):
        raise IndexError(f"index {x} outside shape {shape}")
    c = []
    for s in flatten(shape):
        c.append(x % s)
        x //= s
    return c


def natural_coord(shape: IntTuple, coord) -> List[int]:
    """Accept a 1-D index, a per-mode coordinate (one integer per top-level
    mode, each unravelled colex inside its mode), or a fully natural nested
    coordinate, and return the per-leaf coordinate."""
    if isinstance(coord, int):
        return unravel(shape, coord)
    if not isinstance(shape, tuple):
        # a single mode addressed by a 1-tuple
        if len(coord) != 1:
            raise ValueError("coordinate rank mismatch")
        return natural_coord(shape, coord[0])
    if len(coord) != len(shape):
        raise ValueError(f"coordinate {coord} does not match shape {shape}")
    out: List[int] = []
    for s, c in zip(shape, coord):
        out.extend(natural_coord(s, c))
    return out


def evaluate(L: Layout, coord) -> int:
    """offset = sum over leaves of coordinate times stride ("CUTLASS and CuTe
    layouts", "A layout is a shape and a stride"; 3.5 CUTLASS II, 3.5.3)."""
    c = natural_coord(L.shape, coord)
    return sum(ci * di for ci, di in zip(c, flatten(L.stride)))


def enumerate_offsets(L: Layout) -> List[int]:
    """[L(0), L(1), ..., L(size-1)] by direct evaluation."""
    return [evaluate(L, x) for x in range(size(L))]


def cosize(L: Layout) -> int:
    """Largest offset reached, plus one: the memory footprint (3.5 CUTLASS II,
    3.5.5). Computed by enumeration, the definition itself. READING: a layout
    with an extent of 0 has no coordinates, size 0 and cosize 0."""
    offs = enumerate_offsets(L)
    return max(offs) + 1 if offs else 0


def _nonempty(*Ls: Layout):
    """READING: the algebra (coalesce, composition, complement, divides) is
    defined here for layouts with at least one coordinate."""
    for L in Ls:
        if size(L) == 0:
            raise ValueError("empty layout")


# --------------------------------------------------------------------------
# Construction helpers
# --------------------------------------------------------------------------

def make_colmajor(shape: IntTuple) -> Layout:
    """Compact strides, first leaf fastest: the default "natural" stride
    (3.5 CUTLASS II, 3.5.3 and 3.5.4)."""
    leaves = flatten(shape)
    strides, cur = [], 1
    for s in leaves:
        strides.append(cur)
        cur *= s
    return Layout(shape, _rebuild(shape, strides))


def make_rowmajor(shape: IntTuple) -> Layout:
    """Compact strides, last leaf fastest (3.5 CUTLASS II, 3.5.3, GenRowMajor)."""
    leaves = flatten(shape)
    strides, cur = [0] * len(leaves), 1
    for i in range(len(leaves) - 1, -1, -1):
        strides[i] = cur
        cur *= leaves[i]
    return Layout(shape, _rebuild(shape, strides))


def make_tuple_layout(*modes: Layout) -> Layout:
    """Concatenate layouts as the top-level modes of a new layout."""
    return Layout(tuple(m.shape for m in modes), tuple(m.stride for m in modes))


def _from_leaves(pairs: Sequence[Tuple[int, int]]) -> Layout:
    """One leaf prints as s:d, several as a flat tuple."""
    if len(pairs) == 1:
        return Layout(pairs[0][0], pairs[0][1])
    return Layout(tuple(p[0] for p in pairs), tuple(p[1] for p in pairs))


# --------------------------------------------------------------------------
# Printing / parsing
# --------------------------------------------------------------------------

def _fmt(t: IntTuple) -> str:
    if isinstance(t, tuple):
        return "(" + ",".join(_fmt(x) for x in t) + ")"
    return str(t)


def format_layout(L: Layout) -> str:
    """shape:stride with nested parentheses and no spaces; static-integer
    markers are not printed ("CUTLASS and CuTe layouts", "Results")."""
    return _fmt(L.shape) + ":" + _fmt(L.stride)


def _parse_tuple(s: str, i: int):
    if s[i] == "(":
        items = []
        i += 1
        while True:
            item, i = _parse_tuple(s, i)
            items.append(item)
            if s[i] == ",":
                i += 1
                continue
            if s[i] == ")":
                return tuple(items), i + 1
            raise ValueError(f"bad layout text at {i}: {s!r}")
    j = i
    while j < len(s) and s[j].isdigit():
        j += 1
    if j == i:
        raise ValueError(f"bad layout text at {i}: {s!r}")
    return int(s[i:j]), j


def parse_layout(text: str) -> Layout:
    s = text.replace(" ", "").replace("_", "")
    shape, i = _parse_tuple(s, 0)
    if s[i] != ":":
        raise ValueError(f"missing ':' in {text!r}")
    stride, j = _parse_tuple(s, i + 1)
    if j != len(s):
        raise ValueError(f"trailing text in {text!r}")
    return Layout(shape, stride)


# --------------------------------------------------------------------------
# coalesce
# --------------------------------------------------------------------------

def coalesce(L: Layout) -> Layout:
    """Flatten; drop extent-1 leaves; merge a leaf s1:d1 into its left
    neighbour s0:d0 whenever d1 == s0*d0 ("Layouts as Algebra", "A shape is a
    tree"; 3.5 CUTLASS II, 3.5.6). READING: if nothing is left the result is
    1:0."""
    _nonempty(L)
    pairs = [(s, d) for s, d in zip(flatten(L.shape), flatten(L.stride)) if s != 1]
    out: List[Tuple[int, int]] = []
    for s, d in pairs:
        if out and d == out[-1][0] * out[-1][1]:
            out[-1] = (out[-1][0] * s, out[-1][1])
        else:
            out.append((s, d))
    if not out:
        return Layout(1, 0)
    return _from_leaves(out)


# --------------------------------------------------------------------------
# composition
# --------------------------------------------------------------------------

def compose_function(A: Layout, B: Layout) -> Callable[[int], int]:
    """The definition of A o B: x -> A(B(x)) ("Layouts as Algebra",
    "Composition, worked by hand"; "CUTLASS and CuTe layouts", "A layout is a
    shape and a stride")."""
    return lambda x: evaluate(A, evaluate(B, x))


def _compose_leaf(a_leaves: List[Tuple[int, int]], s: int, d: int) -> List[Tuple[int, int]]:
    """One leaf s:d of B walked through A's coalesced leaves.

    The walk of "Layouts as Algebra", "Composition, worked by hand": a step of
    d through A's domain first skips whole leaves of A that d steps over and
    cuts the leaf it lands inside; then s such steps are laid over the leaves
    that remain, splitting into one result leaf per A-leaf boundary crossed.
    Every cut must be exact, else no layout exists. READING: the walk may not
    run past A's last leaf (B's image must stay inside A's domain).
    """
    if s == 1:
        return [(1, 0)]
    if d == 0:
        return [(s, 0)]
    leaves = list(a_leaves)
    i = 0
    rest = d
    while rest > 1:
        if i >= len(leaves):
            raise NotAdmissible("stride walks past the end of A")
        a, alpha = leaves[i]
        if rest % a == 0:
            rest //= a
            i += 1
        elif a % rest == 0:
            leaves[i] = (a // rest, alpha * rest)
            rest = 1
        else:
            raise NotAdmissible(f"stride {d} does not cut A's leaf {a} exactly")
    out: List[Tuple[int, int]] = []
    rest = s
    while rest > 1:
        if i >= len(leaves):
            raise NotAdmissible("extent walks past the end of A")
        a, alpha = leaves[i]
        if a == 1:
            i += 1
            continue
        if rest % a == 0:
            out.append((a, alpha))
            rest //= a
            i += 1
        elif a % rest == 0:
            out.append((rest, alpha))
            rest = 1
        else:
            raise NotAdmissible(f"extent {s} does not cut A's leaf {a} exactly")
    return out


def compose(A: Layout, B: Layout) -> Layout:
    """A o B as a layout with B's mode tree: each leaf of B becomes a mode of
    the result (a tuple if the walk crossed a boundary of A)."""
    _nonempty(A, B)
    ac = coalesce(A)
    a_leaves = list(zip(flatten(ac.shape), flatten(ac.stride)))

    def go(shape, stride):
        if isinstance(shape, tuple):
            parts = [go(s, d) for s, d in zip(shape, stride)]
            return tuple(p[0] for p in parts), tuple(p[1] for p in parts)
        pairs = _compose_leaf(a_leaves, shape, stride)
        if len(pairs) == 1:
            return pairs[0]
        return tuple(p[0] for p in pairs), tuple(p[1] for p in pairs)

    sh, st = go(B.shape, B.stride)
    R = Layout(sh, st)
    # The walk treats B's leaves one at a time; the definition asks for the
    # whole function. READING: B's image must lie inside A's domain, and the
    # per-leaf results must add up to A(B(x)) at every x (they do not when
    # two leaves of B carry into the same leaf of A). Checked by enumeration.
    n = size(A)
    for x in range(size(B)):
        b = evaluate(B, x)
        if b >= n or evaluate(R, x) != evaluate(A, b):
            raise NotAdmissible(f"A o B is not a layout with B's modes (fails at x={x})")
    return R


# --------------------------------------------------------------------------
# complement
# --------------------------------------------------------------------------

def complement_translates(B: Layout, M: int) -> List[int]:
    """Definition (READING of "the layout of everything B misses", "Layouts
    as Algebra", "Divide is tiling"): the increasing list T of translates with
    T[0] = 0 such that {t + B(x)} covers [0, M) exactly once. Built greedily:
    take the smallest integer not yet covered. Raises NotAdmissible if no such
    tiling exists. Stride-0 leaves of B are ignored (they add no new image)."""
    _nonempty(B)
    if M < 1:
        raise ValueError("complement needs M >= 1")
    kept = [(s, d) for s, d in zip(flatten(B.shape), flatten(B.stride)) if d > 0]
    image = sorted(enumerate_offsets(_from_leaves(kept))) if kept else [0]
    if len(set(image)) != len(image):
        raise NotAdmissible("B visits an offset twice: nothing can tile with it")
    covered = [False] * M
    T: List[int] = []
    u = 0
    while u < M:
        if covered[u]:
            u += 1
            continue
        for v in image:
            w = u + v
            if w >= M or covered[w]:
                raise NotAdmissible(f"translate {u} overflows or overlaps")
            covered[w] = True
        T.append(u)
        u += 1
    return T


def complement(B: Layout, M: int) -> Layout:
    """Closed construction of the complement as a layout: B's leaves with
    stride > 0 and extent > 1 sorted by stride; the gaps between consecutive
    strides become the complement's leaves, and a last leaf runs to M. The
    result is coalesced. Agrees with complement_translates (tested)."""
    _nonempty(B)
    if M < 1:
        raise ValueError("complement needs M >= 1")
    pairs = sorted((d, s) for s, d in zip(flatten(B.shape), flatten(B.stride)) if d > 0 and s > 1)
    out: List[Tuple[int, int]] = []
    cur = 1
    for d, s in pairs:
        if d % cur != 0:
            raise NotAdmissible(f"stride {d} is not a multiple of {cur}")
        out.append((d // cur, cur))
        cur = s * d
    if M % cur != 0 or M < cur:
        raise NotAdmissible(f"B's footprint {cur} does not divide {M}")
    out.append((M // cur, cur))
    return coalesce(_from_leaves(out))


# --------------------------------------------------------------------------
# divides and tiles
# --------------------------------------------------------------------------

Tiler = Union[Layout, int, tuple]


def _tiler_layout(t) -> Layout:
    return t if isinstance(t, Layout) else Layout(t, 1)


def logical_divide(A: Layout, tiler: Tiler) -> Layout:
    """logical_divide(A, B) = A o (B, complement(B, size(A))) ("Layouts as
    Algebra", "Divide is tiling"). Mode 0 addresses inside a tile, mode 1 picks
    the tile ("CUTLASS and CuTe layouts", "A layout is a shape and a stride").

    ``tiler`` is a Layout (divides the whole layout), an int ``b`` (the layout
    b:1), or a tuple with one entry per leading top-level mode of A (divides
    mode by mode; modes past the tuple are kept whole). READING: a tiler whose size does not divide the mode raises
    NotDivisible (3.5 CUTLASS II, 3.5.8)."""
    if isinstance(tiler, tuple):
        if len(tiler) > A.rank:
            raise ValueError(f"tiler {tiler} has {len(tiler)} modes, layout has {A.rank}")
        parts = [logical_divide(A.mode(i), t) for i, t in enumerate(tiler)]
        parts += [A.mode(i) for i in range(len(tiler), A.rank)]
        return make_tuple_layout(*parts)
    B = _tiler_layout(tiler)
    _nonempty(A, B)
    n = size(A)
    if n % size(B) != 0:
        raise NotDivisible(f"tile of size {size(B)} does not divide {n}")
    return compose(A, make_tuple_layout(B, complement(B, n)))


def zipped_divide(A: Layout, tiler: Tiler) -> Layout:
    """The same division with the modes regrouped: all in-tile parts as mode 0,
    all tile-index parts as mode 1 ("CUTLASS and CuTe layouts", "A layout is a
    shape and a stride")."""
    ld = logical_divide(A, tiler)
    if not isinstance(tiler, tuple):
        return ld
    k = len(tiler)
    tiles = [ld.mode(i).mode(0) for i in range(k)]
    rests = [ld.mode(i).mode(1) for i in range(k)] + [ld.mode(i) for i in range(k, ld.rank)]
    return make_tuple_layout(make_tuple_layout(*tiles), make_tuple_layout(*rests))


def _select(t: tuple, step) -> tuple:
    if step is None:
        return t
    return tuple(x for x, keep in zip(t, step) if keep)


def local_tile(A: Layout, tiler: tuple, coord: tuple, step=None) -> Tuple[int, Layout]:
    """One tile of A: divide by the tiler, then fix the tile-index mode at the
    block coordinate ("Layouts as Algebra", "The kernel, in three lines";
    3.5 CUTLASS II, 3.5.6).

    ``coord`` has one entry per tiler mode; ``None`` (CuTe's ``_``) leaves that
    tile-index mode free, and free modes are appended after the tile modes in
    order. ``step`` (a tuple of booleans over the tiler modes, CuTe's Step)
    selects which tiler modes apply to A. Returns (offset, layout): the tile's
    elements are at offset + layout(x)."""
    tiler = _select(tuple(tiler), step)
    coord = _select(tuple(coord), step)
    if len(tiler) != A.rank or len(coord) != len(tiler):
        raise ValueError("local_tile needs one tiler entry and one coordinate per mode")
    zd = zipped_divide(A, tiler)
    tile, rest = zd.mode(0), zd.mode(1)
    offset = 0
    free_modes: List[Layout] = []
    for i, c in enumerate(coord):
        m = rest.mode(i)
        if c is None:
            free_modes.append(m)
        else:
            offset += evaluate(m, c)
    if not free_modes:
        return offset, tile
    modes = [tile.mode(i) for i in range(tile.rank)] + free_modes
    return offset, make_tuple_layout(*modes)


def layout_inverse_coord(thr: Layout, t: int) -> List[int]:
    """The per-mode coordinate c with thr(c) == t, found by search over the
    domain (READING: the thread layout must be a bijection onto [0, size))."""
    hits = [x for x in range(size(thr)) if evaluate(thr, x) == t]
    if len(hits) != 1:
        raise ValueError(f"thread layout is not a bijection at {t}")
    x = hits[0]
    if thr.rank == 1:
        return [x]
    out = []
    for i in range(thr.rank):
        n = size(thr.mode(i))
        out.append(x % n)
        x //= n
    return out


def local_partition(T: Layout, thr: Layout, t: int, step=None) -> Tuple[int, Layout]:
    """Thread t's share of a tile: divide T by the thread layout's shape, then
    fix the in-tile mode at thread t's coordinate and keep the tile-index mode
    ("Layouts as Algebra", "The kernel, in three lines"; 3.5 CUTLASS II,
    3.5.6 and 3.5.7). Thread t's coordinate is the one thr maps to t.
    Returns (offset, layout)."""
    thr_shape = tuple(size(thr.mode(i)) for i in range(thr.rank))
    tcoord = layout_inverse_coord(thr, t)
    if step is not None:
        thr_shape = _select(thr_shape, step)
        tcoord = _select(tuple(tcoord), step)
    zd = zipped_divide(T, thr_shape)
    tile, rest = zd.mode(0), zd.mode(1)
    offset = evaluate(tile, tuple(tcoord))
    return offset, rest


# --------------------------------------------------------------------------
# products and thread-value layouts
# --------------------------------------------------------------------------

def logical_product(A: Layout, B: Layout) -> Layout:
    """READING of "Layouts as Algebra", "Divide is tiling": the product lays
    copies of the tile A out in the pattern B and mirrors the divide
    A o (B, B*). Mode 0 is A itself; mode 1 is B read through the complement
    of A in [0, size(A) * cosize(B)), so copy j of the tile starts where the
    complement puts B(j): (A, complement(A, size(A)*cosize(B)) o B)."""
    _nonempty(A, B)
    return make_tuple_layout(A, compose(complement(A, size(A) * cosize(B)), B))


def product_copies(A: Layout, B: Layout) -> List[List[int]]:
    """The definition of the product spelled out as sets: the translates T of
    A in [0, size(A)*cosize(B)) (complement_translates, the greedy tiling),
    and copy j of A placed at translate T[B(j)]. Returns, per copy j, the
    offsets A(i) + T[B(j)] in i order."""
    T = complement_translates(A, size(A) * cosize(B))
    return [[evaluate(A, i) + T[evaluate(B, j)] for i in range(size(A))] for j in range(size(B))]


def tv_offset(thr: Sequence[int], val: Sequence[int], blocked: Sequence[int], t: Sequence[int],
              v: Sequence[int]) -> int:
    """Offset, in the column-major tile of extents thr[i]*val[i], of value v
    of thread t ("Layouts as Algebra", "The threads are a layout too"). Per
    mode: interleaved, thread t's values are t, t + T, t + 2T, ... (on any
    one step the threads take consecutive offsets); blocked, thread t owns
    the run t*V .. t*V + V - 1. Written out directly, mode by mode."""
    off, scale = 0, 1
    for i in range(len(thr)):
        T, V = thr[i], val[i]
        pos = t[i] * V + v[i] if blocked[i] else t[i] + T * v[i]
        off += pos * scale
        scale *= T * V
    return off
