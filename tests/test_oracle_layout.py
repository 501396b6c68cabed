"""Pins for the layout oracle: the pages' worked values (tests/golden) plus
brute force on tiny layouts. None of these re-types the oracle's formulas;
each compares it with a printed value, a closed form written from a different
place, or an exhaustive enumeration."""

import itertools
import json
import os
import random

import numpy as np
import pytest

from oracle import layout as ol
from oracle.layout import Layout, parse_layout as P

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "layout_pins.json")))


# ---------------------------------------------------------------------------
# Printed worked examples
# ---------------------------------------------------------------------------

def test_zipped_divide_printed_form_and_modes():
    g = GOLD["zipped_divide_256x128"]
    zd = ol.zipped_divide(P(g["layout"]), tuple(g["tiler"]))
    assert str(zd) == g["result"]
    assert str(zd) == g["printed_with_static_markers"].replace("_", "")
    assert str(zd.mode(0)) == g["mode0"]
    assert str(zd.mode(1)) == g["mode1"]


def test_zipped_divide_element_37_44():
    g = GOLD["zipped_divide_256x128"]
    zd = ol.zipped_divide(P(g["layout"]), tuple(g["tiler"]))
    (r, c), (ri, ci), (tr, tc) = g["element"], g["element_in_tile"], g["element_tile"]
    assert (r % 16, c % 16) == (ri, ci) and (r // 16, c // 16) == (tr, tc)
    # natural coordinate ((rowInTile, colInTile), (tileRow, tileCol))
    assert zd(((ri, ci), (tr, tc))) == g["element_offset"]
    assert P(g["layout"])((r, c)) == g["element_offset"]


def test_zipped_divide_equals_hand_tile_index_everywhere():
    """The page's gate: the algebra's map equals the hand-written tile address
    (row = tileRow*16 + rowInTile, col = tileCol*16 + colInTile, index =
    row*128 + col) at all 32,768 elements."""
    g = GOLD["zipped_divide_256x128"]
    zd = ol.zipped_divide(P(g["layout"]), (16, 16))
    n = 0
    for tr, tc, ri, ci in itertools.product(range(16), range(8), range(16), range(16)):
        hand = (tr * 16 + ri) * 128 + (tc * 16 + ci)
        assert zd(((ri, ci), (tr, tc))) == hand
        n += 1
    assert n == g["gate_count"]


def test_divide_identity_tile00():
    """Reading of the 256-index divide-identity gate: mode 0 of the divide at
    tile (0,0) is the matrix itself on its first 16x16 block (256 checks)."""
    A = P("(256,128):(128,1)")
    zd = ol.zipped_divide(A, (16, 16))
    n = 0
    for i, j in itertools.product(range(16), range(16)):
        assert zd(((i, j), (0, 0))) == A((i, j))
        n += 1
    assert n == 256


def test_composition_worked_example():
    g = GOLD["composition_6x2_4x3"]
    A, B = P(g["A"]), P(g["B"])
    assert ol.enumerate_offsets(B) == g["B_values"]
    assert ol.enumerate_offsets(A) == g["A_values"]
    R = ol.compose(A, B)
    assert str(R) == g["R"]
    assert ol.enumerate_offsets(R) == g["R_values"]
    f = ol.compose_function(A, B)
    assert [f(x) for x in range(12)] == g["R_values"]


def test_walkthrough_4x2():
    g = GOLD["walkthrough_4x2"]
    L = P(g["layout"])
    assert L(tuple(g["coord"])) == g["offset"]
    assert ol.size(L) == g["size"] and ol.cosize(L) == g["cosize"]


def test_unravel_4x3():
    g = GOLD["shape_4x3_unravel"]
    L = P(g["layout"])
    assert L(tuple(g["coord"])) == g["offset"]
    assert ol.unravel(L.shape, g["index"]) == g["index_coord"]
    assert L(g["index"]) == g["offset"]


def test_packed_panel():
    g = GOLD["packed_panel"]
    L = P(g["layout"])
    M = g["matrix"]
    # Reading: mode 0 = (row-in-block, col-in-block), mode 1 = (block-row, block-col).
    for r, c in itertools.product(range(4), range(4)):
        assert L(((r % 2, c % 2), (r // 2, c // 2))) == M[r][c]
    # The per-axis (rows, cols) layout of the same panel, per-mode coordinates.
    Lax = P(g["per_axis_layout"])
    for r, c in itertools.product(range(4), range(4)):
        assert Lax((r, c)) == M[r][c]
    assert ol.enumerate_offsets(L) == g["walk"]
    # The page's NumPy view, rebuilt: element strides times the item size.
    a = np.arange(16, dtype=np.int64)
    view = np.lib.stride_tricks.as_strided(a, shape=(2, 2, 2, 2),
                                           strides=np.array(ol.flatten(L.stride)) * a.itemsize)
    assert list(view.strides) == g["numpy_byte_strides_int64"]
    assert view.transpose(2, 0, 3, 1).reshape(4, 4).tolist() == M
    # Row- and column-major readings of the same 16 numbers.
    assert [P(g["row_major"])((r, c)) for r in range(4) for c in range(4)] == list(range(16))
    assert [P(g["col_major"])((r, c)) for c in range(4) for r in range(4)] == list(range(16))


def test_colmajor_rowmajor_points_and_transpose():
    g = GOLD["colmajor_rowmajor_4x6"]
    for key in ("colmajor", "rowmajor"):
        L = P(g[key])
        for coord, off in g[key + "_points"]:
            assert L(tuple(coord)) == off
    assert str(ol.make_colmajor((4, 6))) == g["colmajor"]
    assert str(ol.make_rowmajor((4, 6))) == g["rowmajor"]
    R, T = P(g["rowmajor"]), P(g["transpose_of_rowmajor"])
    for i, j in itertools.product(range(4), range(6)):
        assert R((i, j)) == T((j, i))


def test_nested_2x4_and_coalesce():
    g = GOLD["nested_2x4"]
    L = P(g["layout"])
    assert [[L((i, j)) for j in range(4)] for i in range(2)] == g["rows"]
    assert ol.enumerate_offsets(L) == g["colex_walk"]
    assert str(ol.coalesce(L)) == g["coalesce"]
    assert str(ol.make_colmajor((2, 4))) == g["colmajor"]
    assert str(ol.coalesce(P(g["colmajor"]))) == g["colmajor_coalesce"]
    assert ol.unravel((2, 4), 5) == g["index5_coord"]


def test_costume_24():
    g = GOLD["costume_24"]
    L = P(g["layout"])
    assert ol.enumerate_offsets(L) == list(range(24))
    assert str(ol.coalesce(L)) == g["coalesce"]


def test_divides():
    g = GOLD["divide_8_by_4"]
    assert str(ol.logical_divide(P(g["layout"]), g["tiler"])) == g["result"]
    g = GOLD["colmajor_divide_3x2"]
    assert str(ol.zipped_divide(P(g["layout"]), tuple(g["tiler"]))) == g["result"]


def test_tv_layouts():
    g = GOLD["tv_layouts"]
    good, bad = P(g["coalesced"]), P(g["strided"])
    for t in range(8):
        assert [good((t, v)) for v in range(4)] == [t, t + 8, t + 16, t + 24]
        assert [bad((t, v)) for v in range(4)] == [4 * t + v for v in range(4)]
    # one step v: the 8 threads of the good layout touch 8 consecutive offsets
    for v in range(4):
        offs = sorted(good((t, v)) for t in range(8))
        assert offs == list(range(offs[0], offs[0] + 8))


def test_padding_size_cosize():
    g = GOLD["padding"]
    L = P(g["pad5"])
    assert ol.size(L) == g["pad5_size"] and ol.cosize(L) == g["pad5_cosize"]
    S = P(g["smem33"])
    assert ol.cosize(S) == g["smem33_cosize_by_definition"]
    assert ol.cosize(S) <= g["smem33_allocation_on_page"]
    I = P(g["interleaved"])
    assert sorted(ol.enumerate_offsets(I)) == list(range(32))


def test_cutlass_in_depth_4x8():
    g = GOLD["cutlass_in_depth_4x8"]
    C, R = P(g["colmajor"]), P(g["rowmajor"])
    for i, j in itertools.product(range(4), range(8)):
        assert C((i, j)) == i + 4 * j and R((i, j)) == 8 * i + j


def test_local_tile_shapes():
    # (M,K) row-major A; tile 128x32; block (1, _) keeps the k-tile mode free
    A = ol.make_rowmajor((512, 256))
    off, L = ol.local_tile(A, (128, 32), (1, None))
    assert L.shape == (128, 32, 8)
    assert off == 128 * 256
    # Step projection of an (M,N,K) tiler onto A, B (N,K) and C
    M, N, K = 256, 384, 128
    mA, mB, mC = ol.make_colmajor((M, K)), ol.make_colmajor((N, K)), ol.make_colmajor((M, N))
    tiler, coord = (128, 128, 8), (1, 2, None)
    _, gA = ol.local_tile(mA, tiler, coord, step=(1, 0, 1))
    _, gB = ol.local_tile(mB, tiler, coord, step=(0, 1, 1))
    _, gC = ol.local_tile(mC, tiler, coord, step=(1, 1, 0))
    assert gA.shape == (128, 8, 16) and gB.shape == (128, 8, 16) and gC.shape == (128, 128)


# ---------------------------------------------------------------------------
# Brute force on tiny layouts
# ---------------------------------------------------------------------------

def _random_layout(rng, max_depth=2, max_modes=3, max_extent=4, max_stride=16):
    def node(depth):
        if depth < max_depth and rng.random() < 0.35:
            k = rng.randint(1, 3)
            parts = [node(depth + 1) for _ in range(k)]
            return tuple(p[0] for p in parts), tuple(p[1] for p in parts)
        return rng.randint(1, max_extent), rng.randint(0, max_stride)
    k = rng.randint(1, max_modes)
    parts = [node(1) for _ in range(k)]
    if k == 1 and rng.random() < 0.5:
        return Layout(parts[0][0], parts[0][1])
    return Layout(tuple(p[0] for p in parts), tuple(p[1] for p in parts))


def test_eval_index_equals_eval_unravelled_coordinate():
    rng = random.Random(1)
    for _ in range(300):
        L = _random_layout(rng)
        leaves_s, leaves_d = ol.flatten(L.shape), ol.flatten(L.stride)
        for x in range(ol.size(L)):
            # unravel written out by hand here: digits of x in the mixed radix
            digits, y = [], x
            for s in leaves_s:
                digits.append(y % s)
                y //= s
            assert L(x) == sum(a * b for a, b in zip(digits, leaves_d))


def test_coalesce_preserves_function_and_is_maximal():
    rng = random.Random(2)
    for _ in range(500):
        L = _random_layout(rng)
        C = ol.coalesce(L)
        assert ol.size(C) == ol.size(L)
        assert ol.enumerate_offsets(C) == ol.enumerate_offsets(L)
        s, d = ol.flatten(C.shape), ol.flatten(C.stride)
        if len(s) > 1:
            assert all(x != 1 for x in s)
            assert all(d[i + 1] != s[i] * d[i] for i in range(len(s) - 1))


def test_compose_matches_definition_when_admissible():
    rng = random.Random(3)
    admitted = 0
    for _ in range(3000):
        A = _random_layout(rng, max_stride=8)
        B = _random_layout(rng, max_extent=3, max_stride=6)
        try:
            R = ol.compose(A, B)
        except ol.NotAdmissible:
            continue
        admitted += 1
        assert ol.size(R) == ol.size(B)
        f = ol.compose_function(A, B)
        for x in range(ol.size(B)):
            assert R(x) == f(x)
    assert admitted > 300


def test_compose_with_compact_divisor_layouts_always_admissible():
    """B = (b, n/b):(1, b) with b an exact cut of A's coalesced shape (a
    prefix product times a divisor of the next extent) — what tiling uses —
    must compose, and reproduce A."""
    rng = random.Random(4)
    for _ in range(500):
        A = _random_layout(rng, max_stride=8)
        n = ol.size(A)
        ext = ol.flatten(ol.coalesce(A).shape)
        cuts, pre = set(), 1
        for a in ext:
            cuts |= {pre * r for r in range(1, a + 1) if a % r == 0}
            pre *= a
        b = rng.choice(sorted(cuts))
        B = Layout((b, n // b), (1, b))
        R = ol.compose(A, B)
        assert ol.enumerate_offsets(R) == ol.enumerate_offsets(A)


def test_complement_closed_form_equals_greedy_definition():
    checked = 0
    for s0, s1 in itertools.product(range(1, 5), repeat=2):
        for d0, d1 in itertools.product(range(0, 9), repeat=2):
            B = Layout((s0, s1), (d0, d1))
            for M in (1, 2, 4, 6, 8, 12, 16, 24, 32):
                try:
                    T = ol.complement_translates(B, M)
                except (ol.NotAdmissible, IndexError):
                    T = None
                try:
                    C = ol.complement(B, M)
                except ol.NotAdmissible:
                    C = None
                if T is None:
                    assert C is None, (B, M, C)
                    continue
                assert C is not None, (B, M, T)
                assert ol.enumerate_offsets(C) == T, (B, M)
                checked += 1
    assert checked > 500


def test_complement_plus_b_tiles_exactly():
    rng = random.Random(5)
    for _ in range(400):
        B = _random_layout(rng, max_stride=8)
        for M in (8, 16, 24, 32, 48, 64):
            try:
                C = ol.complement(B, M)
            except ol.NotAdmissible:
                continue
            img = ol.enumerate_offsets(B)
            if len(set(img)) != len(img):
                continue  # B revisits offsets (stride-0 leaves): not a tiling
            hits = sorted(b + c for b in img for c in ol.enumerate_offsets(C))
            assert hits == list(range(M))


@pytest.mark.parametrize("shape,stride,tiler", [
    ((8, 12), (12, 1), (4, 3)),
    ((8, 12), (1, 8), (2, 6)),
    ((16, 6), (6, 1), (8, 2)),
    ((6, 4), (1, 6), (3, 2)),
    ((4, 4), (5, 1), (2, 2)),
])
def test_divide_is_tile_regrouping(shape, stride, tiler):
    A = Layout(shape, stride)
    zd = ol.zipped_divide(A, tiler)
    (bm, bn) = tiler
    for ti, tj, i, j in itertools.product(range(shape[0] // bm), range(shape[1] // bn),
                                          range(bm), range(bn)):
        assert zd(((i, j), (ti, tj))) == A((ti * bm + i, tj * bn + j))


def test_divide_not_divisible():
    with pytest.raises(ol.NotDivisible):
        ol.zipped_divide(Layout((10, 8), (8, 1)), (4, 4))


@pytest.mark.parametrize("shape,stride,tiler", [
    ((8, 12), (12, 1), (4, 3)),
    ((12, 8), (1, 12), (6, 4)),
])
def test_local_tile_enumerates_exact_block(shape, stride, tiler):
    A = Layout(shape, stride)
    bm, bn = tiler
    for ti, tj in itertools.product(range(shape[0] // bm), range(shape[1] // bn)):
        off, L = ol.local_tile(A, tiler, (ti, tj))
        got = sorted(off + L(x) for x in range(ol.size(L)))
        want = sorted(A((ti * bm + i, tj * bn + j)) for i in range(bm) for j in range(bn))
        assert got == want


@pytest.mark.parametrize("thr", ["(4,2):(1,4)", "(4,2):(2,1)", "(2,4):(1,2)"])
def test_local_partition_strided_share(thr):
    T = Layout((8, 8), (8, 1))
    th = P(thr)
    tm, tn = ol.size(th.mode(0)), ol.size(th.mode(1))
    seen = []
    for t in range(8):
        off, L = ol.local_partition(T, th, t)
        # thread t's coordinate inside the thread grid, found by search
        (cm, cn) = next((a, b) for a in range(tm) for b in range(tn) if th((a, b)) == t)
        got = sorted(off + L(x) for x in range(ol.size(L)))
        want = sorted(T((cm + tm * i, cn + tn * j)) for i in range(8 // tm) for j in range(8 // tn))
        assert got == want
        seen += got
    assert sorted(seen) == list(range(64))


def test_parse_format_roundtrip():
    rng = random.Random(6)
    for _ in range(200):
        L = _random_layout(rng)
        assert P(str(L)) == L


def test_rejects_bad_layouts():
    with pytest.raises(ValueError):
        Layout((2, 3), (1,))
    with pytest.raises(ValueError):
        Layout((2, -1), (1, 2))
    with pytest.raises(ValueError):
        Layout((2, 3), (1, -2))
    with pytest.raises(IndexError):
        Layout((2, 3), (1, 2))(6)


def test_empty_layout():
    E = Layout((4, 0), (1, 4))
    assert ol.size(E) == 0 and ol.cosize(E) == 0 and ol.enumerate_offsets(E) == []
    with pytest.raises(IndexError):
        E(0)
    for op in (lambda: ol.coalesce(E), lambda: ol.compose(E, Layout(2, 1)), lambda: ol.complement(E, 8),
               lambda: ol.zipped_divide(E, (2, 2))):
        with pytest.raises(ValueError):
            op()


# ---------------------------------------------------------------------------
# logical_product and thread-value layouts ("Layouts as Algebra", "Divide is
# tiling" and "The threads are a layout too")
# ---------------------------------------------------------------------------

def _compact_layout(rng, max_modes=3, max_extent=4):
    """A compact layout: the extents in a random order, strides the running
    products in that order (a bijection onto [0, size))."""
    k = rng.randint(1, max_modes)
    shape = [rng.randint(1, max_extent) for _ in range(k)]
    order = list(range(k))
    rng.shuffle(order)
    stride, run = [0] * k, 1
    for i in order:
        stride[i] = run
        run *= shape[i]
    return Layout(tuple(shape), tuple(stride)) if k > 1 else Layout(shape[0], stride[0])


def test_tv_builders_reproduce_the_pages_two_layouts():
    """The page's two thread-value layouts for 8 threads and 32 values: the
    interleaved builder gives thread t the values t, t+8, t+16, t+24 and the
    blocked builder the run 4t .. 4t+3 -- value for value the printed
    (8,4):(1,8) and (8,4):(4,1)."""
    g = GOLD["tv_layouts"]
    good, bad = P(g["coalesced"]), P(g["strided"])
    for t in range(8):
        for v in range(4):
            assert ol.tv_offset([8], [4], [0], [t], [v]) == good((t, v))
            assert ol.tv_offset([8], [4], [1], [t], [v]) == bad((t, v))
    # and the product construction yields exactly those printed layouts
    assert str(ol.logical_product(P("8:1"), P("4:1"))) == g["coalesced"]
    swapped = ol.logical_product(P("4:1"), P("8:1"))
    assert str(Layout((swapped.shape[1], swapped.shape[0]), (swapped.stride[1], swapped.stride[0]))) == g["strided"]


def test_logical_product_closed_form_for_compact_tiles():
    """For a compact tile A (a bijection onto [0, size(A))) the copies are
    whole shifted blocks: product(i, j) = A(i) + size(A) * B(j). Mode 0 is A
    itself."""
    rng = random.Random(17)
    checked = 0
    for _ in range(600):
        A = _compact_layout(rng)
        B = _compact_layout(rng) if rng.random() < 0.5 else _random_layout(rng, max_stride=5)
        try:
            R = ol.logical_product(A, B)
        except ol.NotAdmissible:
            # the composition with B needs exact cuts (the composition
            # reading); a compact B always has them
            assert sorted(ol.enumerate_offsets(B)) != list(range(ol.size(B)))
            continue
        checked += 1
        assert R.mode(0) == A
        n = ol.size(A)
        for j in range(ol.size(B)):
            for i in range(n):
                assert R(i + n * j) == A(i) + n * B(j)
    assert checked > 300


def test_logical_product_matches_the_tiling_definition():
    """Any admissible A: copy j of the tile sits at the B(j)-th translate of
    the greedy tiling of [0, size(A)*cosize(B)) by A (complement_translates,
    pinned against the closed complement elsewhere)."""
    rng = random.Random(23)
    checked = 0
    for _ in range(600):
        A = _random_layout(rng, max_modes=2, max_extent=3, max_stride=6)
        B = _random_layout(rng, max_modes=2, max_extent=3, max_stride=4)
        try:
            R = ol.logical_product(A, B)
        except ol.NotAdmissible:
            continue   # no complement, or a composition without exact cuts
        copies = ol.product_copies(A, B)
        n = ol.size(A)
        for j in range(ol.size(B)):
            assert [R(i + n * j) for i in range(n)] == copies[j]
        checked += 1
    assert checked > 100


def test_logical_product_fills_the_holes_of_a_strided_tile():
    """A tile with gaps (2:2 covers 0 and 2): the copies go into the gaps."""
    R = ol.logical_product(P("2:2"), P("2:1"))
    assert str(R) == "(2,2):(2,1)"
    assert ol.product_copies(P("2:2"), P("2:1")) == [[0, 2], [1, 3]]


def test_product_and_divide_are_mirrors():
    """Dividing a product of compact layouts by the tile's size gives back a
    layout with the same values: (tile, which copy)."""
    rng = random.Random(29)
    for _ in range(200):
        A = _compact_layout(rng)
        B = _compact_layout(rng)
        R = ol.logical_product(A, B)
        D = ol.logical_divide(ol.coalesce(R), ol.size(A))
        assert ol.enumerate_offsets(D) == ol.enumerate_offsets(R)
        assert sorted(ol.enumerate_offsets(R)) == list(range(ol.size(A) * ol.size(B)))


def test_product_without_complement_is_caught():
    """Planted mistake: (A, B) without the complement places copies on top of
    each other; the compact closed form catches it."""
    A, B = P("(2,2):(1,2)"), P("3:1")
    wrong = ol.make_tuple_layout(A, B)
    n = ol.size(A)
    assert any(wrong(i + n * j) != A(i) + n * B(j) for j in range(3) for i in range(n))


def test_tv_offset_multi_mode_is_a_bijection_of_the_tile():
    rng = random.Random(31)
    for _ in range(100):
        k = rng.randint(1, 3)
        thr = [rng.randint(1, 4) for _ in range(k)]
        val = [rng.randint(1, 4) for _ in range(k)]
        blk = [rng.randint(0, 1) for _ in range(k)]
        offs = [ol.tv_offset(thr, val, blk, t, v) for t in itertools.product(*[range(x) for x in thr])
                for v in itertools.product(*[range(x) for x in val])]
        assert sorted(offs) == list(range(int(np.prod([a * b for a, b in zip(thr, val)]))))
