"""CPU tests of the C-ABI library: it loads and exports every declared
symbol, its host layout algebra agrees bit-exactly with the oracle, and the
GEMM planner validates and plans without touching a device."""

import ctypes
import itertools
import json
import os
import random
import re

import numpy as np
import pytest

from layout_algebra_tiled_amd import Layout, LtError
from layout_algebra_tiled_amd import _lib as L
from oracle import layout as ol

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "layout_pins.json")))
TILE = json.load(open(os.path.join(ROOT, "tests", "golden", "tile_arithmetic.json")))


def O(lay: Layout) -> ol.Layout:
    """The library's layout as an oracle layout value (same tree, same leaves)."""
    return ol.Layout(lay.shape, lay.stride)


def Lb(x: ol.Layout) -> Layout:
    return Layout.parse(str(x))


def status_of(fn, *a):
    try:
        return fn(*a), None
    except LtError as e:
        return None, e.name
    except (ol.NotAdmissible, ol.NotDivisible, IndexError, ValueError) as e:
        return None, type(e).__name__


# ---------------------------------------------------------------------------
# the library loads and exports the header's functions
# ---------------------------------------------------------------------------

def test_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "lt.h")).read()
    declared = set(re.findall(r"\b(lt_[a-z_0-9]+)\s*\(", header))
    assert declared, "no declarations found"
    lib = L.lib()
    for name in declared:
        assert hasattr(lib, name), f"{name} not exported"
    assert declared == set(L.SIGNATURES), "binding and header disagree"
    assert b"gfx950" in lib.lt_version()


def test_status_strings():
    for code in L.STATUS_NAMES:
        assert L.lib().lt_status_string(code)


# ---------------------------------------------------------------------------
# pins through the library
# ---------------------------------------------------------------------------

def test_pins_through_library():
    g = GOLD["zipped_divide_256x128"]
    zd = Layout.parse(g["layout"]).zipped_divide(g["tiler"])
    assert str(zd) == g["result"]
    assert str(zd.mode(0)) == g["mode0"] and str(zd.mode(1)) == g["mode1"]
    (ri, ci), (tr, tc) = g["element_in_tile"], g["element_tile"]
    assert zd([ri, ci, tr, tc]) == g["element_offset"]          # natural coordinate
    assert zd([ri + 16 * ci, tr + 16 * tc]) == g["element_offset"]  # per-mode coordinate
    assert Layout.parse(g["printed_with_static_markers"]) == zd
    g = GOLD["composition_6x2_4x3"]
    R = Layout.parse(g["A"]).compose(Layout.parse(g["B"]))
    assert str(R) == g["R"] and [R(x) for x in range(12)] == g["R_values"]
    g = GOLD["walkthrough_4x2"]
    W = Layout.parse(g["layout"])
    assert W(g["coord"]) == g["offset"] and W.size() == g["size"] and W.cosize() == g["cosize"]
    g = GOLD["shape_4x3_unravel"]
    assert Layout.parse(g["layout"])(g["index"]) == g["offset"]
    g = GOLD["packed_panel"]
    P = Layout.parse(g["layout"])
    assert [P(x) for x in range(16)] == g["walk"]
    for r, c in itertools.product(range(4), range(4)):
        assert P([r % 2, c % 2, r // 2, c // 2]) == g["matrix"][r][c]
        assert Layout.parse(g["per_axis_layout"])([r, c]) == g["matrix"][r][c]
    assert str(Layout.parse(GOLD["costume_24"]["layout"]).coalesce()) == "24:1"
    assert str(Layout.parse("(2,4):(1,2)").coalesce()) == "8:1"
    assert str(Layout.parse("(2,4):(4,1)").coalesce()) == "(2,4):(4,1)"
    assert str(Layout.parse("8:1").logical_divide(4)) == "(4,2):(1,4)"
    assert str(Layout.parse("(6,4):(1,6)").zipped_divide((3, 2))) == "((3,2),(2,2)):((1,6),(3,12))"
    assert Layout.parse("(4,4):(5,1)").cosize() == 19
    assert Layout.parse("(128,32):(33,1)").cosize() == 4223
    assert str(Layout.colmajor([4, 6])) == "(4,6):(1,4)" and str(Layout.rowmajor([4, 6])) == "(4,6):(6,1)"


# ---------------------------------------------------------------------------
# random layouts: library == oracle
# ---------------------------------------------------------------------------

def _rand(rng, max_depth=2, max_modes=3, max_extent=4, max_stride=16):
    def node(depth):
        if depth < max_depth and rng.random() < 0.35:
            k = rng.randint(1, 3)
            parts = [node(depth + 1) for _ in range(k)]
            return tuple(p[0] for p in parts), tuple(p[1] for p in parts)
        return rng.randint(1, max_extent), rng.randint(0, max_stride)
    k = rng.randint(1, max_modes)
    parts = [node(1) for _ in range(k)]
    if k == 1 and rng.random() < 0.5:
        return ol.Layout(parts[0][0], parts[0][1])
    return ol.Layout(tuple(p[0] for p in parts), tuple(p[1] for p in parts))


def test_eval_size_cosize_coalesce_match_oracle():
    rng = random.Random(10)
    for _ in range(400):
        x = _rand(rng)
        y = Lb(x)
        assert str(y) == str(x)
        assert y.shape == x.shape and y.stride == x.stride
        assert y.size() == ol.size(x) and y.cosize() == ol.cosize(x)
        assert [y(i) for i in range(ol.size(x))] == ol.enumerate_offsets(x)
        assert str(y.coalesce()) == str(ol.coalesce(x))
        for i in range(x.rank):
            assert str(y.mode(i)) == str(x.mode(i))


def test_compose_matches_oracle_including_refusals():
    rng = random.Random(11)
    agree = admitted = 0
    for _ in range(3000):
        a, b = _rand(rng, max_stride=8), _rand(rng, max_extent=3, max_stride=6)
        lib_r, lib_e = status_of(lambda: Lb(a).compose(Lb(b)))
        or_r, or_e = status_of(lambda: ol.compose(a, b))
        assert (lib_e is None) == (or_e is None), (str(a), str(b), lib_e, or_e)
        if lib_e is None:
            admitted += 1
            assert str(lib_r) == str(or_r), (str(a), str(b))
        else:
            assert lib_e == "LT_ERR_NOT_ADMISSIBLE" and or_e == "NotAdmissible"
        agree += 1
    assert admitted > 300


def test_complement_matches_oracle():
    for s0, s1 in itertools.product(range(1, 5), repeat=2):
        for d0, d1 in itertools.product(range(0, 9), repeat=2):
            b = ol.Layout((s0, s1), (d0, d1))
            for M in (1, 4, 6, 8, 12, 16, 24, 32):
                lib_r, lib_e = status_of(lambda: Lb(b).complement(M))
                or_r, or_e = status_of(lambda: ol.complement(b, M))
                assert (lib_e is None) == (or_e is None), (str(b), M)
                if lib_e is None:
                    assert str(lib_r) == str(or_r)


def test_logical_product_matches_oracle_including_refusals():
    rng = random.Random(14)
    admitted = 0
    for _ in range(2000):
        a, b = _rand(rng, max_extent=3, max_stride=6), _rand(rng, max_extent=3, max_stride=4)
        lib_r, lib_e = status_of(lambda: Lb(a).logical_product(Lb(b)))
        or_r, or_e = status_of(lambda: ol.logical_product(a, b))
        assert (lib_e is None) == (or_e is None), (str(a), str(b), lib_e, or_e)
        if lib_e is None:
            admitted += 1
            assert str(lib_r) == str(or_r), (str(a), str(b))
        else:
            assert lib_e in ("LT_ERR_NOT_ADMISSIBLE", "LT_ERR_CAPACITY") and or_e == "NotAdmissible"
    assert admitted > 200


def test_tv_layouts_match_oracle_definition():
    """lt_make_tv_layout against the oracle's direct per-mode definition, and
    the page's two 8-thread layouts through the library."""
    g = GOLD["tv_layouts"]
    assert str(Layout.tv([8], [4])) == g["coalesced"]
    assert str(Layout.tv([8], [4], [1])) == g["strided"]
    rng = random.Random(15)
    for _ in range(200):
        k = rng.randint(1, 3)
        thr = [rng.randint(1, 5) for _ in range(k)]
        val = [rng.randint(1, 5) for _ in range(k)]
        blk = [rng.randint(0, 1) for _ in range(k)]
        tv = Layout.tv(thr, val, blk)
        for t in itertools.product(*[range(x) for x in thr]):
            for v in itertools.product(*[range(x) for x in val]):
                # one integer per top-level mode, unravelled colexicographically
                ti = sum(t[i] * int(np.prod(thr[:i])) for i in range(k))
                vi = sum(v[i] * int(np.prod(val[:i])) for i in range(k))
                got = tv([ti, vi])
                assert got == ol.tv_offset(thr, val, blk, t, v), (thr, val, blk, t, v)


def test_divides_and_tiles_match_oracle():
    rng = random.Random(12)
    shapes = [(8, 12), (12, 8), (16, 6), (6, 16), (4, 4), (24, 8)]
    for _ in range(200):
        m, n = rng.choice(shapes)
        major = rng.choice(["row", "col", "pad"])
        stride = {"row": (n, 1), "col": (1, m), "pad": (n + 3, 1)}[major]
        a = ol.Layout((m, n), stride)
        bm = rng.choice([d for d in range(1, m + 1) if m % d == 0])
        bn = rng.choice([d for d in range(1, n + 1) if n % d == 0])
        assert str(Lb(a).zipped_divide((bm, bn))) == str(ol.zipped_divide(a, (bm, bn)))
        assert str(Lb(a).logical_divide((bm, bn))) == str(ol.logical_divide(a, (bm, bn)))
        tm, tn = rng.randrange(m // bm), rng.randrange(n // bn)
        off, t = Lb(a).local_tile((bm, bn), (tm, tn))
        ooff, ot = ol.local_tile(a, (bm, bn), (tm, tn))
        assert off == ooff and str(t) == str(ot)
        off, t = Lb(a).local_tile((bm, bn), (tm, None))
        ooff, ot = ol.local_tile(a, (bm, bn), (tm, None))
        assert off == ooff and str(t) == str(ot)


def test_local_tile_step_projection_matches_oracle():
    M, N, K = 256, 384, 128
    mA, mB, mC = ol.make_colmajor((M, K)), ol.make_colmajor((N, K)), ol.make_colmajor((M, N))
    tiler, coord = (128, 128, 8), (1, 2, None)
    for lay, step in ((mA, (1, 0, 1)), (mB, (0, 1, 1)), (mC, (1, 1, 0))):
        off, t = Lb(lay).local_tile(tiler, coord, step)
        ooff, ot = ol.local_tile(lay, tiler, coord, step)
        assert off == ooff and str(t) == str(ot)


@pytest.mark.parametrize("tile,thr", [("(8,8):(8,1)", "(4,2):(1,4)"), ("(8,8):(8,1)", "(4,2):(2,1)"),
                                      ("(128,32):(33,1)", "(16,16):(1,16)"), ("(16,8):(1,16)", "(2,4):(1,2)")])
def test_local_partition_matches_oracle(tile, thr):
    T, th = ol.parse_layout(tile), ol.parse_layout(thr)
    for t in range(ol.size(th)):
        off, lay = Lb(T).local_partition(Lb(th), t)
        ooff, olay = ol.local_partition(T, th, t)
        assert off == ooff and str(lay) == str(olay)


def test_local_partition_with_step_matches_oracle():
    sA = ol.Layout((64, 8), (1, 64))       # (BLK_M, BLK_K)
    tC = ol.Layout((16, 16), (1, 16))      # thread grid (THR_M x THR_N)
    for t in (0, 1, 17, 255):
        off, lay = Lb(sA).local_partition(Lb(tC), t, step=(1, 0))
        ooff, olay = ol.local_partition(sA, tC, t, step=(1, 0))
        assert off == ooff and str(lay) == str(olay)


# ---------------------------------------------------------------------------
# error statuses
# ---------------------------------------------------------------------------

def test_error_statuses():
    def err(fn):
        with pytest.raises(LtError) as e:
            fn()
        return e.value.name
    assert err(lambda: Layout.parse("(2,3):(1)")) == "LT_ERR_INVALID_LAYOUT"
    assert err(lambda: Layout.parse("(2,x):(1,2)")) == "LT_ERR_INVALID_ARGUMENT"
    assert Layout.parse("(2,0):(1,2)").size() == 0   # empty, but valid
    assert err(lambda: Layout.parse("(4,3):(3,1)")(12)) == "LT_ERR_OUT_OF_RANGE"
    assert err(lambda: Layout.parse("(4,3):(3,1)")([4, 0])) == "LT_ERR_OUT_OF_RANGE"
    assert err(lambda: Layout.parse("(10,8):(8,1)").zipped_divide((4, 4))) == "LT_ERR_NOT_DIVISIBLE"
    assert err(lambda: Layout.parse("(2,2):(1,1)").complement(8)) == "LT_ERR_NOT_ADMISSIBLE"
    assert err(lambda: Layout.parse("(2,3):(3,1)").compose(Layout.parse("3:1"))) == "LT_ERR_NOT_ADMISSIBLE"
    assert err(lambda: Layout.parse("(65536,65536,65536,65536):(1,1,1,1)").size()) == "LT_ERR_OUT_OF_RANGE"
    big = "(" + ",".join(["2"] * 40) + "):(" + ",".join(["1"] * 40) + ")"
    assert err(lambda: Layout.parse(big)) == "LT_ERR_CAPACITY"


# ---------------------------------------------------------------------------
# capability gate and GEMM planner (no device needed)
# ---------------------------------------------------------------------------

def _desc(ptr, dtype, shape, stride):
    d = L.lt_tensor()
    d.ptr = ptr
    d.dtype = dtype
    d.layout = Layout.make(shape, stride).c
    return d


def _plan(A, B, C, D, bnz=0, kernel=0, split=0, tile_n=0, tile=None, persistent=0):
    o = L.lt_gemm_options()
    o.kernel, o.split_k, o.tile_n, o.persistent = kernel, split, tile_n, persistent
    if tile:
        o.tile_m, o.tile_n = tile
    info = L.lt_gemm_plan_info()
    st = L.lib().lt_gemm_plan(ctypes.byref(A), ctypes.byref(B), ctypes.byref(C) if C else None, ctypes.byref(D),
                              bnz, ctypes.byref(o), ctypes.byref(info))
    return L.STATUS_NAMES[st], info


BASE = 1 << 40   # fake, 256-byte aligned, never dereferenced


def _gemm_descs(M, N, K, dt=L.LT_BF16, a="k", b="k", d="n", off=(0, 0, 0, 0)):
    sz = 2 * (M * K + K * N + 2 * M * N) + 4096
    A = _desc(BASE + off[0], dt, [M, K], [K, 1] if a == "k" else [1, M])
    B = _desc(BASE + sz + off[1], dt, [K, N], [1, K] if b == "k" else [N, 1])
    C = _desc(BASE + 2 * sz + off[2], dt, [M, N], [N, 1] if d == "n" else [1, M])
    D = _desc(BASE + 3 * sz + off[3], dt, [M, N], [N, 1] if d == "n" else [1, M])
    return A, B, C, D


def test_arch_gate_refuses_before_launch():
    lib = L.lib()
    A, B, C, D = _gemm_descs(256, 256, 64)
    try:
        lib.lt_set_arch_override(b"gfx942")
        buf = ctypes.create_string_buffer(32)
        assert L.STATUS_NAMES[lib.lt_device_check(buf, 32)] == "LT_ERR_ARCH_MISMATCH"
        assert buf.value == b"gfx942"
        st = lib.lt_gemm_run(ctypes.byref(A), ctypes.byref(B), None, ctypes.byref(D), 1.0, 0.0, None, None, 0, None)
        assert L.STATUS_NAMES[st] == "LT_ERR_ARCH_MISMATCH"
        lay = Layout.parse("(4,4):(4,1)")
        st = lib.lt_layout_eval_device(ctypes.byref(lay.c), 0x1000, 16, None)
        assert L.STATUS_NAMES[st] == "LT_ERR_ARCH_MISMATCH"
        lib.lt_set_arch_override(b"gfx950")
        assert L.STATUS_NAMES[lib.lt_device_check(buf, 32)] == "LT_OK"
    finally:
        lib.lt_set_arch_override(None)


def test_plan_kernel_choice_for_the_workloads():
    st, i = _plan(*_gemm_descs(256, 128, 64, L.LT_F16))
    assert st == "LT_OK" and i.kernel == L.LT_KERNEL_WAVE16 and i.grid == (16 * 8) // 4
    st, i = _plan(*_gemm_descs(4096, 4096, 4096, L.LT_F16), bnz=1)
    assert st == "LT_OK" and i.kernel == L.LT_KERNEL_TILED and i.grid == 256
    st, i = _plan(*_gemm_descs(8192, 8192, 8192))
    assert st == "LT_OK" and i.kernel == L.LT_KERNEL_TILED and (i.tiles, i.grid, i.persistent) == (1024, 1024, 0)
    assert (i.tile_m, i.tile_n) == (256, 256) and i.tile_k in (32, 64) and i.waves in (4, 8)
    assert i.waves * i.wave_m * i.wave_n == 256 * 256 and i.stages >= 2
    st, i = _plan(*_gemm_descs(32, 8192, 8192))
    assert st == "LT_OK" and i.kernel == L.LT_KERNEL_SKINNY and i.split_k == 1 and i.grid == 256
    st, i = _plan(*_gemm_descs(32, 1024, 8192))
    assert st == "LT_OK" and i.kernel == L.LT_KERNEL_SKINNY and i.split_k == 8
    assert i.workspace_bytes == 8 * 32 * 1024 * 4


def test_plan_tiled_needs_32bit_copy_offsets():
    """The 256x256 kernel addresses a K slice as a uniform base plus per-lane
    32-bit byte offsets; a leading dimension that pushes the last row past
    4 GiB goes to the 16x16 kernel instead (still a valid plan)."""
    M = N = K = 256
    ok = ((1 << 31) - 64) // (M - 1)   # ((M-1)*lda + BK)*2 just under 4 GiB
    for lda, expect in ((K, L.LT_KERNEL_TILED), (ok - 64, L.LT_KERNEL_TILED), (ok + 64, L.LT_KERNEL_WAVE16)):
        A = _desc(BASE, L.LT_BF16, [M, K], [lda, 1])
        B = _desc(BASE + (1 << 36), L.LT_BF16, [K, N], [1, K])
        D = _desc(BASE + (2 << 36), L.LT_BF16, [M, N], [N, 1])
        st, i = _plan(A, B, None, D)
        assert st == "LT_OK" and i.kernel == expect, (lda, st, i.kernel)
    # the same limit on an N-major B: (BK-1)*ldb + N elements
    B = _desc(BASE + (1 << 36), L.LT_BF16, [K, N], [1 << 26, 1])
    A = _desc(BASE, L.LT_BF16, [M, K], [K, 1])
    D = _desc(BASE + (2 << 36), L.LT_BF16, [M, N], [N, 1])
    st, i = _plan(A, B, None, D)
    assert st == "LT_OK" and i.kernel == L.LT_KERNEL_WAVE16
    st, i = _plan(A, B, None, D, kernel=L.LT_KERNEL_TILED)
    assert st == "LT_ERR_NOT_DIVISIBLE" or st == "LT_ERR_UNSUPPORTED"


def test_plan_closed_forms_reproduce_page_arithmetic():
    """The closed forms behind the plan's LDS bill and MFMA count reproduce the
    pages' printed tile arithmetic, then give the plan's own figures."""
    def stage_bytes(bm, bn, bk, elem):
        return (bm * bk + bk * bn) * elem

    def instr_per_wave(wm, wn, wk, im, in_, ik):
        return (wm // im) * (wn // in_) * (wk // ik)

    s = TILE["smem_bill"]
    assert stage_bytes(128, 128, 32, 2) == s["tile_128x128x32_fp16_bytes_per_stage"]
    assert 2 * stage_bytes(128, 128, 32, 2) == s["two_stages"]
    assert 3 * stage_bytes(128, 128, 32, 2) == s["three_stages"]
    assert 3 * stage_bytes(128, 256, 64, 2) == s["tile_128x256x64_three_stages"]
    assert stage_bytes(128, 64, 32, 2) == s["tile_128x64x32_fp16_bytes_per_stage"]
    m = TILE["mma_count"]
    assert instr_per_wave(64, 64, 32, 16, 8, 8) == m["instr_16x8x8"]
    assert instr_per_wave(64, 64, 32, 16, 8, 16) == m["instr_16x8x16"]
    t = TILE["tile_intensity"]
    assert stage_bytes(128, 128, 64, 2) == t["bytes_per_step"]
    assert 2 * 128 * 128 * 64 == t["flops_per_step"] and t["flops_per_step"] // t["bytes_per_step"] == 64
    w = TILE["wave_quantisation"]
    assert (4096 // 128) ** 2 == w["tiles_128x128"] and round(w["tiles_128x128"] / w["sms"], 2) == w["waves_128x128"]
    assert round(w["tiles_128x256"] / w["sms"], 2) == w["waves_128x256"]
    _, i = _plan(*_gemm_descs(8192, 8192, 8192))
    # the stages, plus 32 KiB beside them where the epilogue stages D
    assert i.lds_bytes == i.stages * stage_bytes(i.tile_m, i.tile_n, i.tile_k, 2) + 32 * 1024
    assert (i.mfma_m, i.mfma_n, i.mfma_k) in ((32, 32, 16), (16, 16, 32))
    assert i.mfma_per_wave_kstep == instr_per_wave(i.wave_m, i.wave_n, i.tile_k, i.mfma_m, i.mfma_n, i.mfma_k)
    assert i.tiles / 256 == 4.0   # 1,024 tiles on 256 CUs: whole waves


def test_plan_validation_statuses():
    # misaligned base
    A, B, C, D = _gemm_descs(256, 256, 64, off=(2, 0, 0, 0))
    assert _plan(A, B, C, D)[0] == "LT_ERR_MISALIGNED_OPERAND"
    # leading dimension not a multiple of 8 elements
    A = _desc(BASE, L.LT_F16, [256, 60], [60, 1])
    _, B, C, D = _gemm_descs(256, 256, 60, L.LT_F16)
    assert _plan(A, B, C, D)[0] == "LT_ERR_MISALIGNED_OPERAND"
    # no unit stride
    A = _desc(BASE, L.LT_F16, [64, 64], [128, 2])
    _, B, C, D = _gemm_descs(64, 64, 64, L.LT_F16)
    assert _plan(A, B, C, D)[0] == "LT_ERR_UNSUPPORTED"
    # shape mismatch
    A, _, C, D = _gemm_descs(256, 256, 64)
    B = _desc(BASE + (1 << 30), L.LT_BF16, [128, 256], [1, 128])
    assert _plan(A, B, C, D)[0] == "LT_ERR_INVALID_ARGUMENT"
    # dtype mix
    A, B, C, D = _gemm_descs(256, 256, 64)
    A.dtype = L.LT_F16
    assert _plan(A, B, C, D)[0] == "LT_ERR_UNSUPPORTED"
    # a ragged shape: the tiled kernel takes it when forced (edge tiles are
    # predicated); the automatic choice keeps a problem smaller than one tile
    # on the 16x16 kernel
    A, B, C, D = _gemm_descs(250, 256, 64)
    st, i = _plan(A, B, C, D, kernel=L.LT_KERNEL_TILED)   # one 256x256 tile = four 128x128 ones
    assert st == "LT_OK" and i.kernel == L.LT_KERNEL_TILED and (i.tile_m, i.tile_n, i.grid) == (128, 128, 4)
    st, i = _plan(A, B, C, D, kernel=L.LT_KERNEL_TILED, tile_n=256)
    assert st == "LT_OK" and (i.tile_n, i.grid) == (256, 1)
    # block tiles other than 256x256 and 256x128 are refused, and so is a
    # split of 256x128 tiles
    assert _plan(A, B, C, D, kernel=L.LT_KERNEL_TILED, tile_n=64)[0] == "LT_ERR_UNSUPPORTED"
    assert _plan(A, B, C, D, kernel=L.LT_KERNEL_TILED, tile_n=128, split=2)[0] == "LT_ERR_UNSUPPORTED"
    assert _plan(A, B, C, D)[1].kernel == L.LT_KERNEL_WAVE16
    # K-major operands copy whole 16-byte chunks of K: K % 8 != 0 is refused
    A = _desc(BASE, L.LT_BF16, [256, 60], [64, 1])
    B = _desc(BASE + (1 << 30), L.LT_BF16, [60, 256], [1, 64])
    D = _desc(BASE + (2 << 30), L.LT_BF16, [256, 256], [256, 1])
    assert _plan(A, B, None, D, kernel=L.LT_KERNEL_TILED)[0] == "LT_ERR_NOT_DIVISIBLE"
    assert _plan(A, B, None, D)[1].kernel == L.LT_KERNEL_WAVE16
    # D overlapping A
    A, B, C, D = _gemm_descs(256, 256, 64)
    D.ptr = A.ptr + 64
    assert _plan(A, B, C, D)[0] == "LT_ERR_INVALID_ARGUMENT"
    # D == C exactly is allowed
    A, B, C, D = _gemm_descs(256, 256, 64)
    C.ptr = D.ptr
    assert _plan(A, B, C, D, bnz=1)[0] == "LT_OK"
    # beta != 0 needs C
    assert _plan(A, B, None, D, bnz=1)[0] == "LT_ERR_INVALID_ARGUMENT"
    # workspace check before the device is touched
    A, B, C, D = _gemm_descs(32, 1024, 8192)
    st = L.lib().lt_gemm_run(ctypes.byref(A), ctypes.byref(B), None, ctypes.byref(D), 1.0, 0.0, None, None, 0, None)
    assert L.STATUS_NAMES[st] == "LT_ERR_WORKSPACE"
    # a workspace that is big enough but not 256-byte aligned is refused too
    ws = _plan(A, B, None, D)[1].workspace_bytes
    assert ws > 0
    st = L.lib().lt_gemm_run(ctypes.byref(A), ctypes.byref(B), None, ctypes.byref(D), 1.0, 0.0, None,
                             ctypes.c_void_p(BASE + (5 << 30) + 64), ws, None)
    assert L.STATUS_NAMES[st] == "LT_ERR_WORKSPACE"


def test_plan_ragged_shapes_on_the_tiled_kernel():
    """Ragged M, N and K plan onto the 256x256 kernel with a ceil-divided tile
    grid when padding to whole tiles adds at most half again."""
    for (M, N, K), expect in (((1000, 1304, 1000), L.LT_KERNEL_TILED), ((4000, 4000, 4000), L.LT_KERNEL_TILED),
                              ((296, 296, 296), L.LT_KERNEL_WAVE16), ((8192, 8200, 8192), L.LT_KERNEL_TILED)):
        st, i = _plan(*_gemm_descs(M, N, K))
        assert st == "LT_OK" and i.kernel == expect, (M, N, K, st, i.kernel)
        if expect == L.LT_KERNEL_TILED:
            tiles = -(-M // i.tile_m) * -(-N // i.tile_n)
            assert i.tiles == tiles and i.grid == tiles - i.sk_tiles + i.sk_workgroups


def _tile_plan(M, N, K, split=0, want_n=0):
    """The planner's rule, written out, in K-slice times of a 256x128 tile:
    256x256 tiles cost 2 per slice; their whole rounds of 256 tiles stay
    data-parallel and the last round's rem tiles are split into S K segments
    when that saves 3 % (12 slices per partial the last segment reads back,
    plus 24 when all 256x128 tiles fit one round) or when forced;
    256x128 tiles cost 23/20 per slice and are never split; 128x128 tiles
    cost 16/20 per slice, never split, taken only by a fully automatic tile
    choice. Returns (tile code: 256, 128 for 256x128, 64 for 128x128,
    data-parallel tiles, split tiles, S)."""
    kt = -(-K // 64)
    n256 = -(-M // 256) * -(-N // 256)
    n128 = -(-M // 256) * -(-N // 128)
    rem, S = n256 % 256, 1
    c256 = -(-n256 // 256) * kt * 2
    if split == 0:
        if rem:
            S = min(256 // rem, 8, kt // 4)
            if S >= 2:
                t_split = (n256 // 256 * kt + -(-kt // S) + 12 * (S - 1) + (24 if n128 <= 256 else 0)) * 2
                if 100 * t_split < 97 * c256:
                    c256 = t_split
                else:
                    S = 1
    elif split > 1:
        S = min(split, kt)
        rem = rem or min(n256, 256)
    if S < 2:
        S, rem = 1, 0
    n128 = -(-M // 256) * -(-N // 128)
    c128 = -(-n128 // 256) * kt * 23
    n64 = -(-M // 128) * -(-N // 128)
    if want_n == 0 and split <= 1 and (S < 2 or 2 * n64 >= 256) and -(-n64 // 256) * kt * 16 < min(c128, c256 * 20):
        return 64, n64, 0, 1   # 128x128 tiles (tile_n 128, tile_m 128)
    if want_n == 128 or (want_n == 0 and split <= 1 and c128 < c256 * 20):
        return 128, n128, 0, 1
    return 256, n256 - rem, rem, S


def test_plan_tile_choice_and_split_remainder():
    for (M, N, K, split) in ((6144, 4096, 2048, 0), (4096, 4096, 4096, 0), (8192, 8192, 8192, 0),
                             (512, 768, 512, 0), (512, 512, 640, 2), (2048, 2048, 64, 0), (4096, 4352, 1024, 0),
                             (8192, 8192, 8192, 1), (512, 512, 512, 1), (512, 512, 128, 0), (1792, 1792, 7040, 0),
                             (2048, 2048, 8192, 0), (8192, 8448, 8192, 0), (300, 520, 200, 0), (6144, 4096, 2048, 1)):
        st, i = _plan(*_gemm_descs(M, N, K), kernel=L.LT_KERNEL_TILED, split=split)
        assert st == "LT_OK" and i.kernel == L.LT_KERNEL_TILED, (M, N, K, st)
        tn, dp, rem, S = _tile_plan(M, N, K, split)
        sq = tn == 64   # 128x128 tiles
        # tiles run persistent (one workgroup per CU) when 256 rows high and
        # whole, K a multiple of 64 with at least 4 slices, more than 256 of
        # them, and for 256x256 tiles no split remainder (beta = 0 here)
        pers = (not sq and M % 256 == 0 and N % tn == 0 and K % 64 == 0 and K >= 256 and dp > 256 and rem == 0
                and (tn == 128 or K <= 4096))
        grid = 256 if pers else dp + rem * S
        want = (128 if sq else 256, 128 if sq else tn, rem, S, grid, int(pers))
        assert (i.tile_m, i.tile_n, i.sk_tiles, i.split_k, i.grid, i.persistent) == want, \
            (M, N, K, i.tile_m, i.tile_n, i.sk_tiles, i.split_k, i.grid, i.persistent, want)
        assert i.tiles == dp + rem
        assert i.sk_workgroups == rem * S
        want_ws = ((rem * 4 + 255) // 256 * 256 + rem * S * 256 * 256 * 4) if rem else 0
        assert i.workspace_bytes == want_ws
    # the 6144x4096x2048 workload: 384 256x256 tiles = 1.5 rounds, and K is
    # too short (32 slices) for the split to pay; 768 256x128 tiles fill
    # three whole rounds, walked by 256 persistent workgroups, with or
    # without C
    st, i = _plan(*_gemm_descs(6144, 4096, 2048, a="m", b="n"))
    assert (i.tile_n, i.sk_tiles, i.tiles, i.grid, i.persistent) == (128, 0, 768, 256, 1)
    A, B, C, D = _gemm_descs(6144, 4096, 2048, a="m", b="n")
    st, i = _plan(A, B, C, D, bnz=1)
    assert st == "LT_OK" and (i.tile_n, i.tiles, i.grid, i.persistent) == (128, 768, 256, 1)
    # 8192^3: 1,024 256x256 tiles are four whole rounds, one per workgroup
    # (128 slices: past the persistent launch's range for 256x256 tiles);
    # at K = 4096 256 persistent workgroups walk them (beta = 0), with
    # beta != 0 one workgroup per tile
    st, i = _plan(*_gemm_descs(8192, 8192, 8192))
    assert (i.tile_n, i.sk_tiles, i.tiles, i.grid, i.persistent) == (256, 0, 1024, 1024, 0)
    st, i = _plan(*_gemm_descs(8192, 8192, 4096))
    assert (i.tile_n, i.sk_tiles, i.tiles, i.grid, i.persistent) == (256, 0, 1024, 256, 1)
    A, B, C, D = _gemm_descs(8192, 8192, 4096)
    st, i = _plan(A, B, C, D, bnz=1)
    assert (i.tile_n, i.sk_tiles, i.tiles, i.grid, i.persistent) == (256, 0, 1024, 1024, 0)
    # 49 256x256 tiles of 110 slices: a 5-way split would pay 4 partials'
    # read-back (measured 84.9 us), 98 whole 256x128 tiles half the CUs
    # (78.3 us); 196 128x128 tiles take 49.5 us
    st, i = _plan(*_gemm_descs(1792, 1792, 7040))
    assert (i.tile_m, i.tile_n, i.sk_tiles, i.split_k, i.grid, i.persistent) == (128, 128, 0, 1, 196, 0)
    # 2560^3: 400 128x128 tiles need two rounds; 200 256x128 tiles one (38.6
    # us against 43.4)
    st, i = _plan(*_gemm_descs(2560, 2560, 2560))
    assert (i.tile_m, i.tile_n, i.grid) == (256, 128, 200)
    # 64 256x256 tiles of 128 slices: 256 128x128 tiles (63.0 us) beat 128
    # whole 256x128 tiles (87-91 us) and 4 segments each (91-92 us); 16
    # tiles of 256 slices split 8 ways (128 workgroups, 83.7 us) beat 64
    # 128x128 tiles (92.4 us)
    st, i = _plan(*_gemm_descs(2048, 2048, 8192))
    assert (i.tile_m, i.tile_n, i.sk_tiles, i.split_k, i.grid) == (128, 128, 0, 1, 256)   # 63.0 us
    st, i = _plan(*_gemm_descs(1024, 1024, 16384))
    assert (i.tile_n, i.sk_tiles, i.split_k, i.grid) == (256, 16, 8, 128)
    # 1,056 tiles: four whole rounds and 32 tiles split 8 ways (a 4 % saving)
    st, i = _plan(*_gemm_descs(8192, 8448, 8192))
    assert (i.tile_n, i.sk_tiles, i.split_k, i.grid) == (256, 32, 8, 1024 + 256)


def test_plan_persistent_option():
    """persistent = 2 forces the persistent launch (grid min(tiles, 256)),
    refused (LT_ERR_UNSUPPORTED) for ragged tiles, K not a multiple of 64 or
    fewer than 4 slices, and for 256x256 tiles with beta != 0 or a split
    remainder; 1 turns it off; other values are invalid."""
    def plan(M, N, K, pers, tile_n=128):
        return _plan(*_gemm_descs(M, N, K), kernel=L.LT_KERNEL_TILED, tile=(256, tile_n), persistent=pers)
    st, i = plan(2048, 2048, 320, 2)
    assert st == "LT_OK" and (i.persistent, i.grid, i.tiles) == (1, 128, 128)
    st, i = plan(4864, 2176, 512, 2)
    assert st == "LT_OK" and (i.persistent, i.grid, i.tiles) == (1, 256, 323)
    st, i = plan(6144, 4096, 2048, 1)
    assert st == "LT_OK" and (i.persistent, i.grid) == (0, 768)
    st, i = plan(6144, 4096, 2048, 0)
    assert st == "LT_OK" and (i.persistent, i.grid) == (1, 256)
    for M, N, K in ((2000, 2048, 256), (2048, 2000, 256), (2048, 2048, 200), (2048, 2048, 192)):
        assert plan(M, N, K, 2)[0] == "LT_ERR_UNSUPPORTED", (M, N, K)
        assert plan(M, N, K, 0)[1].persistent == 0
    assert plan(2048, 2048, 256, 3)[0] == "LT_ERR_INVALID_ARGUMENT"
    # 256x256 tiles (beta = 0, no split remainder): chosen past one round
    st, i = plan(2048, 2048, 256, 2, tile_n=256)
    assert st == "LT_OK" and (i.persistent, i.grid, i.tiles, i.tile_n) == (1, 64, 64, 256)
    assert plan(2048, 2048, 256, 0, tile_n=256)[1].persistent == 0
    assert plan(8192, 8192, 4096, 0, tile_n=256)[1].persistent == 1
    assert plan(8192, 8192, 8192, 0, tile_n=256)[1].persistent == 0
    assert plan(8192, 8192, 8192, 2, tile_n=256)[1].persistent == 1
    A, B, C, D = _gemm_descs(2048, 2048, 256)
    assert _plan(A, B, C, D, bnz=1, kernel=L.LT_KERNEL_TILED, tile=(256, 256), persistent=2)[0] == "LT_ERR_UNSUPPORTED"
    # 1,056 tiles leave a split remainder: no persistent launch
    assert plan(8192, 8448, 8192, 2, tile_n=256)[0] == "LT_ERR_UNSUPPORTED"


def test_plan_m_major_output_is_transposed():
    st, i = _plan(*_gemm_descs(512, 256, 128, d="m"))
    assert st == "LT_OK" and i.kernel == L.LT_KERNEL_TILED   # solved as D^T = B^T A^T


def test_empty_problem_is_a_no_op():
    A, B, C, D = _gemm_descs(0, 256, 64)
    st = L.lib().lt_gemm_run(ctypes.byref(A), ctypes.byref(B), None, ctypes.byref(D), 1.0, 0.0, None, None, 0, None)
    assert L.STATUS_NAMES[st] == "LT_OK"


def test_empty_layout_matches_oracle():
    E = Layout.parse("(4,0):(1,4)")
    assert E.size() == 0 and E.cosize() == 0
    with pytest.raises(LtError):
        E(0)
    for op in (lambda: E.coalesce(), lambda: E.compose(Layout.parse("2:1")), lambda: E.complement(8),
               lambda: E.zipped_divide((2, 2))):
        with pytest.raises(LtError) as e:
            op()
        assert e.value.name == "LT_ERR_INVALID_LAYOUT"


def test_plan_unit_mode_prefers_a_real_unit_stride():
    """An (8,1) operand stored (1,8): the stride-1 mode is mode 0, so the
    extent-1 mode's stride does not need to be a multiple of 8."""
    A = _desc(BASE, L.LT_F16, [16, 8], [8, 1])
    B = _desc(BASE + 4096, L.LT_F16, [8, 1], [1, 8])
    D = _desc(BASE + 8192, L.LT_F16, [16, 1], [8, 1])
    st, i = _plan(A, B, None, D)
    assert st == "LT_OK"


def test_fused_epilogue_argument_checks_before_the_device():
    A, B, C, D = _gemm_descs(256, 256, 64)
    bad = L.lt_epilogue(None, 1, 0, 7, None)
    st = L.lib().lt_gemm_run_ex(ctypes.byref(A), ctypes.byref(B), None, ctypes.byref(D), 1.0, 0.0, None,
                                ctypes.byref(bad), None, 0, None)
    assert L.STATUS_NAMES[st] == "LT_ERR_INVALID_ARGUMENT"
    neg = L.lt_epilogue(None, -2, 0, L.LT_ACT_RELU, None)
    st = L.lib().lt_gemm_run_ex(ctypes.byref(A), ctypes.byref(B), None, ctypes.byref(D), 1.0, 0.0, None,
                                ctypes.byref(neg), None, 0, None)
    assert L.STATUS_NAMES[st] == "LT_ERR_INVALID_ARGUMENT"


def test_plan_reports_the_wave_layout_of_the_data_parallel_launch():
    """The data-parallel launch runs 4 waves (one per SIMD) for every operand
    major-ness: 256x256 tiles as 128x128 wave tiles (8 x 8 MFMA blocks x 2 K
    steps per wave per 64-deep K slice, 2 stages of 64 KiB), 256x128 tiles as
    128x64 wave tiles (8 x 4 blocks, 3 stages of 48 KiB). With K-major A and
    B the epilogue stages D beside the stages (32 KiB of the 160 beside 128,
    16 beside 144), which the LDS figure includes."""
    for a, b in (("k", "k"), ("m", "k"), ("k", "n"), ("m", "n")):
        staged = a == "k" and b == "k"
        st, i = _plan(*_gemm_descs(2048, 2048, 1024, a=a, b=b), kernel=L.LT_KERNEL_TILED, tile_n=256, split=1)
        assert st == "LT_OK" and i.kernel == L.LT_KERNEL_TILED, (a, b, st)
        assert (i.waves, i.wave_m, i.wave_n) == (4, 128, 128), (a, b)
        assert (i.tile_m, i.tile_n, i.tile_k, i.stages) == (256, 256, 64, 2)
        assert i.mfma_per_wave_kstep == 8 * 8 * 2 and (i.mfma_m, i.mfma_n, i.mfma_k) == (16, 16, 32)
        assert i.lds_bytes == 2 * 2 * 256 * 64 * 2 + (32 * 1024 if staged else 0), (a, b)
        st, i = _plan(*_gemm_descs(2048, 2048, 1024, a=a, b=b), kernel=L.LT_KERNEL_TILED, tile_n=128)
        assert st == "LT_OK" and (i.waves, i.wave_m, i.wave_n) == (4, 128, 64), (a, b)
        assert (i.tile_m, i.tile_n, i.tile_k, i.stages, i.grid) == (256, 128, 64, 3, 128)
        assert i.mfma_per_wave_kstep == 8 * 4 * 2
        assert i.lds_bytes == 3 * (256 + 128) * 64 * 2 + (16 * 1024 if staged else 0), (a, b)


def test_plan_persistent_with_c_needs_c_rows_within_32_bit_copy_offsets():
    """The persistent launch with C copies 16 rows of C per copy instruction
    through a 32-bit byte offset: a C row stride of 2^27 elements or more
    leaves the planner's choice on one workgroup per tile and refuses the
    forced persistent launch; 2^27 - 8 is still taken."""
    for ldc, ok in ((2 ** 27 - 8, True), (2 ** 27, False)):
        A, B, C, D = _gemm_descs(6144, 4096, 2048)
        C = _desc(BASE + (1 << 44), L.LT_BF16, [6144, 4096], [ldc, 1])
        st, i = _plan(A, B, C, D, bnz=1, kernel=L.LT_KERNEL_TILED, tile_n=128)
        assert st == "LT_OK" and i.persistent == (1 if ok else 0), (ldc, st)
        st, i = _plan(A, B, C, D, bnz=1, kernel=L.LT_KERNEL_TILED, tile_n=128, persistent=2)
        assert st == ("LT_OK" if ok else "LT_ERR_UNSUPPORTED"), (ldc, st)


def test_plan_tile_order():
    """The data-parallel launch's tile order: super-blocks where the
    last-level-cache model says they pay (measured faster on these shapes),
    the raster where they do not (measured slower or even), the raster with
    odd rounds walking K downward where a round's 32 panels exceed 192 MiB
    (K above 12288), 0 for the persistent launch; forcing super-blocks needs
    tile counts in multiples of 16 and whole, unsplit tiles, forcing the
    K-reversed raster K a multiple of 64 and more than one round."""
    for (M, N, K), want in (((16384, 16384, 8192), 2), ((12288, 12288, 12288), 2), ((16384, 8192, 8192), 2),
                            ((16384, 16384, 12288), 2), ((8192, 8192, 8192), 1), ((8192, 28672, 8192), 1),
                            ((16384, 16384, 16384), 3), ((12288, 12288, 16384), 3), ((8192, 8192, 4096), 0)):
        st, i = _plan(*_gemm_descs(M, N, K))
        assert st == "LT_OK" and i.tile_order == want, (M, N, K, i.tile_order)
        assert (i.persistent == 1) == (want == 0)
    descs = _gemm_descs(4096, 8192, 512)
    for order in (1, 2, 3):
        o = L.lt_gemm_options()
        o.kernel, o.tile_n, o.persistent, o.tile_order = L.LT_KERNEL_TILED, 256, 1, order
        info = L.lt_gemm_plan_info()
        st = L.lib().lt_gemm_plan(*(ctypes.byref(d) for d in descs[:2]), None, ctypes.byref(descs[3]), 0,
                                  ctypes.byref(o), ctypes.byref(info))
        assert L.STATUS_NAMES[st] == "LT_OK" and info.tile_order == order
    o = L.lt_gemm_options()
    o.kernel, o.tile_n, o.persistent, o.tile_order = L.LT_KERNEL_TILED, 256, 1, 2
    for M, N, K in ((4096, 4096 + 256, 512), (1024, 1024, 16384)):   # 17 tile columns; a split plan
        d = _gemm_descs(M, N, K)
        st = L.lib().lt_gemm_plan(ctypes.byref(d[0]), ctypes.byref(d[1]), None, ctypes.byref(d[3]), 0,
                                  ctypes.byref(o), ctypes.byref(L.lt_gemm_plan_info()))
        assert L.STATUS_NAMES[st] == "LT_ERR_UNSUPPORTED", (M, N, K)
    o.tile_order = 3
    for M, N, K in ((4096, 4096, 512), (4096, 8192, 520)):   # one round; a partial K slice
        d = _gemm_descs(M, N, K)
        st = L.lib().lt_gemm_plan(ctypes.byref(d[0]), ctypes.byref(d[1]), None, ctypes.byref(d[3]), 0,
                                  ctypes.byref(o), ctypes.byref(L.lt_gemm_plan_info()))
        assert L.STATUS_NAMES[st] == "LT_ERR_UNSUPPORTED", (M, N, K)
    o.tile_order = 4
    st = L.lib().lt_gemm_plan(*(ctypes.byref(d) for d in descs[:2]), None, ctypes.byref(descs[3]), 0,
                              ctypes.byref(o), ctypes.byref(L.lt_gemm_plan_info()))
    assert L.STATUS_NAMES[st] == "LT_ERR_INVALID_ARGUMENT"


def test_plan_lds_of_persistent_and_split_launches():
    """The persistent launches stage D for every major-ness (256x256 beside
    128 KiB: +32 KiB; 256x128 with or without C: +16 KiB, which the launch
    with C shares with C rows 192..255), and a launch of split segments only
    holds just its stages."""
    for a, b in (("k", "k"), ("m", "n")):
        st, i = _plan(*_gemm_descs(6144, 4096, 2048, a=a, b=b), kernel=L.LT_KERNEL_TILED, tile_n=128,
                      persistent=2)
        assert st == "LT_OK" and i.persistent == 1 and i.lds_bytes == 160 * 1024, (a, b, st)
        st, i = _plan(*_gemm_descs(6144, 4096, 2048, a=a, b=b), bnz=1, kernel=L.LT_KERNEL_TILED,
                      tile_n=128, persistent=2)
        assert st == "LT_OK" and i.persistent == 1 and i.lds_bytes == 160 * 1024, (a, b, st)
        st, i = _plan(*_gemm_descs(8192, 8192, 2048, a=a, b=b), kernel=L.LT_KERNEL_TILED, tile_n=256,
                      persistent=2)
        assert st == "LT_OK" and i.persistent == 1 and i.lds_bytes == 160 * 1024, (a, b, st)
    st, i = _plan(*_gemm_descs(1024, 1024, 16384), kernel=L.LT_KERNEL_TILED, tile_n=256)
    assert st == "LT_OK" and i.grid == i.sk_workgroups > 0, i.as_dict()   # every tile split
    assert i.lds_bytes == 2 * 2 * 256 * 64 * 2


def test_noalloc_refuses_oversized_plans_before_the_device():
    """lt_gemm_run_noalloc refuses a plan whose scratch exceeds its static
    array (a forced 8-way split of 256 tiles: 512 MiB of partials) with
    LT_ERR_WORKSPACE before touching the device, and every automatic plan of
    the tiled and skinny kernels fits it."""
    A, B, C, D = _gemm_descs(8192, 8192, 8192)
    o = L.lt_gemm_options()
    o.split_k = 8
    st = L.lib().lt_gemm_run_noalloc(ctypes.byref(A), ctypes.byref(B), None, ctypes.byref(D), 1.0, 0.0,
                                     ctypes.byref(o), None, None)
    assert L.STATUS_NAMES[st] == "LT_ERR_WORKSPACE"
    for M, N, K in ((256, 256, 65536), (1792, 1792, 7040), (2304, 2304, 4096), (32, 64, 65536), (32, 8192, 8192),
                    (7936, 8192, 8192)):
        st, i = _plan(*_gemm_descs(M, N, K))
        assert st == "LT_OK" and i.workspace_bytes <= L.LT_NOALLOC_SCRATCH_BYTES, (M, N, K, i.workspace_bytes)

def test_oversized_explicit_layout_is_refused_before_the_library():
    """An explicit layout that reaches past the tensor's storage is refused by
    the binding (the C ABI sees only a pointer)."""
    import torch
    from layout_algebra_tiled_amd import gemm as g
    t = torch.empty(100, dtype=torch.float16)
    with pytest.raises(ValueError):
        g.tensor_desc(t, Layout.make([10, 20], [20, 1]))
    g.tensor_desc(t, Layout.make([10, 10], [10, 1]))          # exactly fits
    with pytest.raises(ValueError):
        g.tensor_desc(t[50:], Layout.make([10, 10], [10, 1]))  # the view starts 50 elements in
