"""Address trace of the tiled kernel's global-to-LDS copy against the oracle.

The copy map in tiled_config.hpp (Operand::stored_chunk and Operand::offset,
compiled here for the host) is traced for every wave, lane and copy
instruction of an operand, and compared with the same map built from the
oracle's layout algebra, independently of the kernel's code:

  * the copy's thread-value layout is the interleaved one of "Layouts as
    Algebra", "The threads are a layout too" (oracle tv_offset): instruction
    v of the workgroup fills LDS chunks 64 v .. 64 v + 63, lane by lane;
  * the LDS tile stores logical chunk (row, c) at the swizzled position the
    kernel's design states (inverted here by search, not by assuming the
    swizzle is an involution);
  * the chunk's source is the operand's block tile from oracle local_tile,
    the three-line kernel of "Layouts as Algebra", "The kernel, in three
    lines": local_tile(mA, (BM, BK), (tm, _)) gives (BM, BK, k-tile) with the
    K tile free, evaluated at the chunk's (row, k) and K slice.

READING (the pages do not treat ragged edges): a block tile that reaches
past the operand's last row reads, for those rows, the last row (K-major) or
the last 8-element chunk of M/N (M/N-major) instead: valid memory whose
products land only in outputs that are never stored. Parity is bit-exact on
every copy, ragged tiles included.
"""

import os
import subprocess

import pytest

from oracle import layout as ol
from tests.proc import skip_if_gpu_initialised

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "layout_algebra_tiled_amd", "csrc")

BM, BK = 256, 64
ROWS = {(0, "a"): 256, (0, "b"): 256, (1, "a"): 256, (1, "b"): 128, (2, "a"): 256, (2, "b"): 256}
NWAVES = {0: 4, 1: 4, 2: 8}


@pytest.fixture(scope="module")
def tracer(tmp_path_factory):
    skip_if_gpu_initialised()
    d = tmp_path_factory.mktemp("trace")
    exe = d / "trace"
    subprocess.check_call(["g++", "-std=c++17", "-O1", f"-I{CSRC}", "-o", str(exe),
                           os.path.join(ROOT, "tests", "native", "operand_trace.cpp")])

    def run(cases):
        text = "".join(f"{c} {op} {k} {ld} {rows} {row0}\n" for c, op, k, ld, rows, row0 in cases)
        out = subprocess.run([str(exe)], input=text, capture_output=True, text=True, check=True).stdout.split("\n")
        res = []
        for i in range(0, 2 * len(cases), 2):
            _, opi, nw, bk, ksb = out[i].split()
            vals = [int(x) for x in out[i + 1].split()]
            res.append({"OPI": int(opi), "NW": int(nw), "BK": int(bk), "KSLICE": int(ksb),
                        "copies": list(zip(vals[0::2], vals[1::2]))})
        return res

    return run


# --- the LDS tile: logical chunk (row, c) -> stored chunk ------------------

def ktile_stored(row, c):
    """K-major tile: rows of BK elements, C = BK/8 chunks of 16 bytes; chunk c
    of row r is stored at position c XOR ((r // R) mod C) of its row, R = 16/C
    rows per 256-byte window."""
    C = BK // 8
    R = 16 // C
    return C * row + (c ^ ((row // R) % C))


def mntile_stored(W):
    """M/N-major tile: BK rows of K, W chunks of 8 M/N elements each; chunk c
    of K row r is stored at c XOR (4 (r mod 4) + 2 ((r div 8) mod 2))."""
    def at(krow, c):
        return W * krow + (c ^ (4 * (krow & 3) + 2 * ((krow >> 3) & 1)))
    return at


def stored_to_logical(kmaj, rows):
    """Invert the stored position by search over every logical chunk."""
    if kmaj:
        C = BK // 8
        pairs = {ktile_stored(r, c): (r, c) for r in range(rows) for c in range(C)}
        assert len(pairs) == rows * C
    else:
        W = rows // 8
        at = mntile_stored(W)
        pairs = {at(r, c): (r, c) for r in range(BK) for c in range(W)}
        assert len(pairs) == BK * W
    return pairs


def operand_layout(kmaj, rows_pad, K, ld):
    """The operand as a (rows, K) layout: A is M x K, B is taken as N x K.
    K-major: element (r, k) at r*ld + k; M/N-major: at k*ld + r."""
    return ol.Layout((rows_pad, K), (ld, 1) if kmaj else (1, ld))


def expected_offsets(kmaj, rows, row0, K, ld, kt, nwaves, opi, ROWSZ):
    """Byte offset (from the operand base) of every copy, in the tracer's
    (wave, lane, i) order, for K slice kt, from the oracle."""
    rows_pad = -(-max(rows, row0 + ROWSZ) // ROWSZ) * ROWSZ
    L = operand_layout(kmaj, rows_pad, K, ld)
    off0, tile = ol.local_tile(L, (ROWSZ, BK), (row0 // ROWSZ, None))
    inv = stored_to_logical(kmaj, ROWSZ)
    last_row_off, last_tile = ol.local_tile(L, (ROWSZ, BK), ((rows - 1) // ROWSZ, None))
    out = []
    for w in range(nwaves):
        for lane in range(64):
            for i in range(opi):
                q = ol.tv_offset((64,), (nwaves * opi,), (0,), (lane,), (w * opi + i,))
                r, c = inv[q]
                if kmaj:
                    row, kk = r, 8 * c
                    if row0 + row >= rows:    # READING: clamp to the last row
                        e = last_row_off + ol.evaluate(last_tile, ((rows - 1) % ROWSZ, kk, kt))
                    else:
                        e = off0 + ol.evaluate(tile, (row, kk, kt))
                else:
                    m, kk = 8 * c, r
                    if row0 + m + 8 > rows:   # READING: clamp to the last 8-element chunk
                        e = ol.evaluate(L, (rows - 8, kt * BK + kk))
                    else:
                        e = off0 + ol.evaluate(tile, (m, kk, kt))
                out.append(2 * e)
    return out


CASES = [
    # (cfg, operand, K-major, ld, rows of the operand, block tile index, K, K slices to check)
    (0, "a", 1, 520, 1000, 0, 512, (0, 1, 7)),
    (0, "a", 1, 520, 1000, 3, 512, (0, 7)),      # ragged: rows 1000..1023 clamp
    (0, "a", 0, 1024, 1000, 0, 512, (0, 5)),
    (0, "a", 0, 1024, 1000, 3, 512, (0, 7)),     # ragged M-major: chunks past 992 clamp
    (0, "b", 1, 584, 600, 2, 576, (0, 8)),
    (0, "b", 0, 608, 600, 2, 576, (0, 8)),
    (1, "b", 1, 520, 600, 4, 512, (0, 7)),       # 128-wide B tile
    (1, "b", 0, 640, 600, 4, 512, (0, 7)),
    (1, "a", 0, 1024, 1000, 1, 512, (2,)),
    (2, "a", 1, 520, 1000, 3, 512, (0, 7)),      # 8 waves
    (2, "b", 0, 608, 600, 1, 512, (0, 3)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"cfg{c[0]}-{c[1]}-{'k' if c[2] else 'mn'}-t{c[5]}")
def test_copy_addresses_match_the_algebra(tracer, case):
    cfg, op, kmaj, ld, rows, tile, K, slices = case
    ROWSZ = ROWS[(cfg, op)]
    row0 = tile * ROWSZ
    (res,) = tracer([(cfg, op, kmaj, ld, rows, row0)])
    nw, opi = res["NW"], res["OPI"]
    assert nw == NWAVES[cfg] and res["BK"] == BK
    assert opi * nw * 1024 == ROWSZ * BK * 2     # the copies cover the slice once
    stored = [q for q, _ in res["copies"]]
    # every LDS chunk of the slice is written exactly once, in lane-linear
    # 1 KiB runs per instruction
    assert sorted(stored) == list(range(ROWSZ * BK * 2 // 16))
    for kt in slices:
        got = [off + kt * res["KSLICE"] for _, off in res["copies"]]
        exp = expected_offsets(kmaj, rows, row0, K, ld, kt, nw, opi, ROWSZ)
        bad = [(j, g, e) for j, (g, e) in enumerate(zip(got, exp)) if g != e]
        assert not bad, (case, kt, bad[:5])


def test_partial_first_slice_addresses(tracer):
    """K not a multiple of BK: the kernel shifts the K range to start at
    kbase = K - KT*BK < 0 (the host moves the operand base by kbase), so
    slice kt covers k = kbase + kt*BK .. ; a copy whose chunk lies at k < 0
    in slice 0 is not loaded. Every loaded copy reads element (row, k) of the
    operand's plain layout."""
    K, rows, ld = 500, 1000, 520
    KT = -(-K // BK)
    kbase = K - KT * BK
    for kmaj in (1, 0):
        ldx = ld if kmaj else 1024
        (res,) = tracer([(0, "a", kmaj, ldx, rows, 0)])
        L = operand_layout(kmaj, 1024, K, ldx)
        inv = stored_to_logical(kmaj, 256)
        shift = 2 * kbase * (1 if kmaj else ldx)       # the host's base move, in bytes
        for kt in (0, 1, KT - 1):
            for q, off in res["copies"]:
                r, c = inv[q]
                row, kk = (r, 8 * c) if kmaj else (8 * c, r)
                k = kbase + kt * BK + kk
                if k < 0:
                    assert kt == 0
                    continue
                assert shift + off + kt * res["KSLICE"] == 2 * ol.evaluate(L, (row, k)), (kmaj, kt, q)


def test_trace_catches_a_wrong_swizzle_reading(tracer):
    """The comparison is sharp: with the M/N-major swizzle's row term read
    as 4 (r mod 4) alone, the trace disagrees."""
    (res,) = tracer([(0, "a", 0, 1024, 1000, 0)])
    W = 32
    wrong = {W * r + (c ^ (4 * (r & 3))): (r, c) for r in range(BK) for c in range(W)}
    right = stored_to_logical(0, 256)
    L = operand_layout(0, 1024, 512, 1024)
    off0, tile = ol.local_tile(L, (256, BK), (0, None))
    mism = 0
    for q, off in res["copies"]:
        r, c = wrong[q]
        mism += off != 2 * (off0 + ol.evaluate(tile, (8 * c, r, 0)))
        r, c = right[q]
        assert off == 2 * (off0 + ol.evaluate(tile, (8 * c, r, 0)))
    assert mism > 0


@pytest.mark.parametrize("cfg,op,kmaj,ld", [(1, "a", 1, 520), (1, "b", 1, 584), (1, "a", 0, 4096), (1, "b", 0, 640),
                                            (0, "a", 1, 1032), (0, "b", 0, 2048)])
def test_persistent_offsets_are_row0_offsets_plus_a_tile_base(tracer, cfg, op, kmaj, ld):
    """The persistent launch copies an interior tile through the offsets of a
    tile at row 0 plus a uniform tile base: for every copy, the offset the
    per-tile launch computes for a tile starting at row0 equals the row-0
    offset plus the element offset of (row0, k = 0) in the operand's
    layout (oracle evaluate), times two bytes."""
    ROWSZ = ROWS[(cfg, op)]
    rows = 16 * ROWSZ
    (r0,) = tracer([(cfg, op, kmaj, ld, ROWSZ, 0)])
    L = operand_layout(kmaj, rows, 64, ld)
    for t in (1, 5, 15):
        row0 = t * ROWSZ
        (rt,) = tracer([(cfg, op, kmaj, ld, rows, row0)])
        base = 2 * ol.evaluate(L, (row0, 0))
        assert [q for q, _ in rt["copies"]] == [q for q, _ in r0["copies"]]
        assert all(o1 == base + o0 for (_, o1), (_, o0) in zip(rt["copies"], r0["copies"])), (cfg, op, kmaj, t)
