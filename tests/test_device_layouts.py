"""The tiled kernel's compile-time layouts (device_layout.hpp, compiled for
the host) checked on the CPU: swizzles are bijections, the copy's
thread-value layout fetches exactly what the swizzle stores, fragment reads of
16 (or 32) lanes hit distinct LDS banks, and the transposed-read addressing,
run through the read semantics measured on gfx950, hands every lane its MFMA
fragment. The unswizzled maps are also compared with the host layout algebra."""

import os
import subprocess

from tests.proc import skip_if_gpu_initialised

import pytest

from layout_algebra_tiled_amd import Layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "layout_algebra_tiled_amd", "csrc")


@pytest.fixture(scope="module")
def maps(tmp_path_factory):
    skip_if_gpu_initialised()
    d = tmp_path_factory.mktemp("devlayout")
    exe = d / "dump"
    subprocess.check_call(["g++", "-std=c++17", "-O1", f"-I{CSRC}", "-o", str(exe),
                           os.path.join(ROOT, "tests", "native", "device_layout_dump.cpp")])
    out = subprocess.check_output([str(exe)], text=True).split("\n")
    m, i = {}, 0
    while i < len(out):
        head = out[i].split()
        if not head:
            i += 1
            continue
        m[tuple(head)] = [int(x) for x in out[i + 1].split()]
        i += 2
    return m


def _ktile(maps, bk):
    key = next(k for k in maps if k[0] == "ktile" and k[1] == str(bk))
    C = int(key[2])
    v = maps[key]
    return C, lambda row, c: v[row * C + c]


@pytest.mark.parametrize("bk", [32, 64])
def test_ktile_swizzle_is_bijection_and_row_local(maps, bk):
    C, at = _ktile(maps, bk)
    allv = [at(r, c) for r in range(256) for c in range(C)]
    assert sorted(allv) == list(range(256 * C))
    for r in range(256):   # a row's chunks stay in that row
        assert sorted(at(r, c) for c in range(C)) == list(range(r * C, (r + 1) * C))
    # the unswizzled chunk layout is (C,256):(1,C) of the layout algebra, and
    # the swizzle XORs the chunk with the row's 256-byte window index mod C
    L = Layout.parse(f"({C},256):(1,{C})")
    R = 16 // C
    for r in range(256):
        for c in range(C):
            assert L([c, r]) == C * r + c
            assert at(r, c) == C * r + (c ^ ((r // R) % C))


@pytest.mark.parametrize("bk", [32, 64])
def test_ktile_fragment_reads_conflict_free(maps, bk):
    """16 consecutive lanes read 16 consecutive rows at one logical chunk:
    their 16-byte chunks must fall in 16 distinct 16-byte bank groups of a
    256-byte (64-bank) window."""
    C, at = _ktile(maps, bk)
    for r0 in range(0, 256, 16):
        for c in range(C):
            groups = {at(r0 + i, c) % 16 for i in range(16)}
            assert len(groups) == 16, (bk, r0, c)


@pytest.mark.parametrize("bk", [32, 64])
def test_copy_fetches_what_swizzle_stores(maps, bk):
    """Stored chunk q receives logical (row, chunk) with at(row, chunk) == q;
    the kernel's inversion (at(row, q % C) - C*row) gives exactly that."""
    C, at = _ktile(maps, bk)
    inv = {at(r, c): (r, c) for r in range(256) for c in range(C)}
    for q in range(256 * C):
        row = q // C
        lchunk = at(row, q % C) - C * row
        assert inv[q] == (row, lchunk)


def _mntile(maps, w=32):
    v = maps[("mntile", "64", str(w))]
    return v, (lambda k, c: v[k * w + c])


@pytest.mark.parametrize("w", [32, 16])
def test_mntile_bijection(maps, w):
    v, at = _mntile(maps, w)
    assert sorted(v) == list(range(64 * w))
    for k in range(64):   # each K row keeps its own w chunks
        assert sorted(at(k, c) for c in range(w)) == list(range(w * k, w * (k + 1)))
        for c in range(w):   # an involution inside the row
            assert at(k, at(k, c) - w * k) - w * k == c


@pytest.mark.parametrize("mf,w", [(32, 32), (16, 32), (16, 16)])
def test_transposed_reads_hand_each_lane_its_fragment(maps, mf, w):
    """The M/N-major operand path: lanes address the LDS tile (K rows of 8*w
    elements: 256 for a 256-wide block tile, 128 for a 128-wide one) as the
    kernel does, the read semantics measured on gfx950 are applied, and every
    lane must receive the MFMA fragment of its row and K values; each 32-lane
    half must touch 32 distinct 8-byte bank pairs (no LDS bank conflict)."""
    _, at = _mntile(maps, w)
    width = 8 * w
    kstep = 512 // mf
    tr = maps[("mtr", str(mf))]
    krow0 = [tr[3 * l] for l in range(64)]
    krow1 = [tr[3 * l + 1] for l in range(64)]
    col = [tr[3 * l + 2] for l in range(64)]
    lds = {}
    for k in range(64):
        for mn in range(width):
            lds[at(k, mn // 8) * 16 + (mn % 8) * 2] = (k, mn)
    bases = [b for b in ((0, 32, 96, 224) if mf == 32 else (0, 16, 48, 112, 240)) if b + mf <= width]
    for s in range(64 // kstep):          # K step
        for base in bases:
            for q, krow in ((0, krow0), (1, krow1)):
                addr = []
                for l in range(64):
                    k = krow[l] + kstep * s
                    mn = base + col[l]
                    addr.append(at(k, mn // 8) * 16 + (mn % 8) * 2)
                for h in (0, 32):
                    pairs = {(a % 256) // 8 for a in addr[h:h + 32]}
                    assert len(pairs) == 32, (mf, s, base, q, h)
                for l in range(64):
                    g, i = l // 16, l % 16
                    for e in range(4):
                        src = 16 * g + 4 * e + i // 4
                        k, mn = lds[addr[src] + 2 * (i % 4)]
                        assert k == kstep * s + 8 * (l // mf) + 4 * q + e
                        assert mn == base + 16 * (g % (mf // 16)) + i


@pytest.mark.parametrize("mf", [32, 16])
def test_mfma_operand_and_output_maps(maps, mf):
    """Operand: lane l reads row l % MF, K chunk l // MF of the step (the
    layout (MF, 64/MF):(1, MF)); output: the lanes' registers cover the MF x MF
    block once, column = lane % MF, and registers 4g..4g+3 of a lane are four
    consecutive rows (the epilogue's 8-byte stores)."""
    key = next(k for k in maps if k[0] == "mfrag" and k[1] == str(mf))
    kstep, nacc = int(key[2]), int(key[3])
    assert kstep == 512 // mf and nacc == mf * mf // 64
    fr = maps[key]
    L = Layout.parse(f"({mf},{64 // mf}):(1,{mf})")
    for l in range(64):
        row, chunk, flat = fr[3 * l], fr[3 * l + 1], fr[3 * l + 2]
        assert (row, chunk) == (l % mf, l // mf)
        assert flat == L(l) == row + mf * chunk
    out = maps[("mout", str(mf))]
    cells = set()
    for l in range(64):
        rows = [out[2 * (nacc * l + v)] for v in range(nacc)]
        for v in range(nacc):
            assert out[2 * (nacc * l + v) + 1] == l % mf
            cells.add((rows[v], l % mf))
        for g in range(nacc // 4):
            assert rows[4 * g:4 * g + 4] == list(range(rows[4 * g], rows[4 * g] + 4))
    assert cells == {(r, c) for r in range(mf) for c in range(mf)}


def _staged(maps, cpr):
    unit = maps[("staged_unit", str(cpr), "128")]
    sl = maps[("staged_slot", str(cpr), "128")]
    return (lambda r, u: unit[r * 2 * cpr + u]), (lambda r, q: sl[2 * (r * cpr + q)]), \
        (lambda r, q: sl[2 * (r * cpr + q) + 1])


def _distinct_banks(addrs, nbytes, window):
    """LDS accesses of nbytes each, served together: no two touch the same
    4-byte bank of a window-byte (window/4-bank) LDS."""
    banks = [(a % window) // 4 + k for a in addrs for k in range(nbytes // 4)]
    return len(set(banks)) == len(banks)


@pytest.mark.parametrize("cpr", [8, 16])
def test_staged_store_round_trip_and_banks(maps, cpr):
    """The staged D store, rows of a wave tile 8*cpr columns wide (64 or 128)
    in the layout of dev::StagedRows. The map covers 128 rows once in 8-byte
    units; slot(r, q) holds units 2q and 2q+1 of row r (swapped when the map
    says so). One pass (32 rows): the accumulators' 8-byte writes (row =
    lane % 16 of the 16x16 block, four consecutive columns) are bank-free
    whether the LDS serves 16 lanes (128 bytes) or 32 (256 bytes) per cycle,
    the 16-byte reads whether it serves 8 lanes or 16, and the lane that
    reads chunk q of row r gets exactly row r, columns 8q .. 8q+7, which it
    stores there."""
    unit, slot, swapped = _staged(maps, cpr)
    RB = 16 * cpr
    allu = [unit(r, u) for r in range(128) for u in range(2 * cpr)]
    assert sorted(allu) == [8 * i for i in range(128 * 2 * cpr)]
    for r in range(128):
        for q in range(cpr):
            lo, hi = (unit(r, 2 * q + 1), unit(r, 2 * q)) if swapped(r, q) else (unit(r, 2 * q), unit(r, 2 * q + 1))
            assert (lo, hi) == (slot(r, q), slot(r, q) + 8)
    out = maps[("mout", "16")]
    orow = lambda l, v: out[2 * (4 * l + v)]   # the block's N index (four consecutive columns)
    ocol = lambda l: out[2 * (4 * l) + 1]      # the block's M index
    byte_of = {}
    for bi in range(2):
        for j in range(cpr // 2):
            addrs = []
            for l in range(64):
                r, n0 = 16 * bi + ocol(l), orow(l, 0)
                assert [orow(l, v) for v in range(4)] == [n0 + v for v in range(4)]
                a = unit(r, (2 * (16 * j + n0)) >> 3)
                for v in range(4):
                    assert a + 2 * v not in byte_of
                    byte_of[a + 2 * v] = (r, 16 * j + n0 + v)
                addrs.append(a)
            for g in range(4):
                assert _distinct_banks(addrs[16 * g:16 * g + 16], 8, 128)
            for h in range(2):
                assert _distinct_banks(addrs[32 * h:32 * h + 32], 8, 256)
    assert len(byte_of) == 32 * RB // 2
    for k in range(32 * RB // 1024):
        addrs = []
        for l in range(64):
            r, q = (64 * k + l) // cpr, (64 * k + l) % cpr
            a = slot(r, q)
            got = [byte_of[a + 2 * e] for e in range(8)]
            if swapped(r, q):   # the reader swaps the two 8-byte halves back
                got = got[4:] + got[:4]
            assert got == [(r, 8 * q + e) for e in range(8)]
            addrs.append(a)
        for g in range(8):
            assert _distinct_banks(addrs[8 * g:8 * g + 8], 16, 128)
        for g in range(4):
            assert _distinct_banks(addrs[16 * g:16 * g + 16], 16, 256)


def test_staged_c_tile_copy_and_reads(maps):
    """The C tile of the staged store with C (256-byte rows, dev::StagedC):
    the direct-to-LDS copy writing slot pos of row r fetches the chunk the
    map stores there, the map covers the tile once, and the accumulators'
    8-byte C reads of a half-wave (two units of 16 rows) reach 64 distinct
    banks of a 256-byte window."""
    c = maps[("staged_c", "16", "128")]
    at = lambda r, q: c[2 * (r * 16 + q)]
    chunk_at = lambda r, pos: c[2 * (r * 16 + pos) + 1]
    assert sorted(at(r, q) for r in range(128) for q in range(16)) == [16 * i for i in range(128 * 16)]
    for r in range(128):
        for pos in range(16):
            assert at(r, chunk_at(r, pos)) == 256 * r + 16 * pos
    out = maps[("mout", "16")]
    orow = lambda l: out[2 * (4 * l)]
    ocol = lambda l: out[2 * (4 * l) + 1]
    for i in range(8):
        for j in range(8):
            addrs = []
            for l in range(64):
                r, cb = 16 * i + ocol(l), 2 * (16 * j + orow(l))
                addrs.append(at(r, cb >> 4) + (cb & 15))
            for h in range(2):
                assert _distinct_banks(addrs[32 * h:32 * h + 32], 8, 256)


def test_fragment_and_accumulator_maps(maps):
    frag = maps[("frag",)]
    assert frag == [(l % 32) + 32 * (l // 32) for l in range(64)]
    acc = maps[("acc",)]
    cells = set()
    for l in range(64):
        for v in range(16):
            r, c = acc[2 * (16 * l + v)], acc[2 * (16 * l + v) + 1]
            assert c == l % 32
            cells.add((r, c))
    assert cells == {(r, c) for r in range(32) for c in range(32)}
    copy = maps[("copy",)]
    assert copy == list(range(256))


def test_kernel_thread_value_maps_are_the_library_products(maps):
    """The copy's (lane, instruction) -> stored chunk map and the MFMA operand
    fragments (lane -> (row, K chunk)) are built in device code by the
    interleaved thread-value builder; the host library builds the same
    layouts through complement and composition (lt_make_tv_layout)."""
    copy = maps[("copy",)]
    tv = Layout.tv([64], [4])
    assert copy == [tv(l + 64 * i) for i in range(4) for l in range(64)]
    frag = maps[("frag",)]
    tv32 = Layout.tv([32], [2])
    assert frag == [tv32(l) for l in range(64)]
    for mf in (16, 32):
        key = next(k for k in maps if k[0] == "mfrag" and k[1] == str(mf))
        fr = maps[key]
        tvm = Layout.tv([mf], [64 // mf])
        assert [fr[3 * l + 2] for l in range(64)] == [tvm(l) for l in range(64)]
        # the same fragment in element space of the column-major (MF, KSTEP)
        # operand atom: lanes (MF rows, 64/MF K groups) x 8 values along K,
        # blocked in the K mode
        el = Layout.tv([mf, 64 // mf], [1, 8], [0, 1])
        for l in range(64):
            for v in range(8):
                row, kk = l % mf, 8 * (l // mf) + v
                assert el([l, v]) == row + mf * kk
