"""Checks on the gfx950 machine code of the built library (CPU only: the code
objects are extracted from liblt.so and disassembled with the ROCm LLVM
tools).

1. Every tiled-kernel variant is present as device code with a host-side
   launch stub, so no configuration the planner can pick is missing.
2. The transposing LDS reads of M/N-major operands land in registers some
   time after they issue. For each such read, every control-flow path from it
   must retire it with an `s_waitcnt lgkmcnt(N)` before any instruction names
   one of its destination registers (a read of them would see stale data, a
   write would be overwritten when the load lands). LDS operations retire in
   order, so lgkmcnt(N) retires the read once N or more LDS operations were
   issued after it on that path (with a scalar load in between, which may
   retire out of order, only lgkmcnt(0) counts).
3. The tiled kernels' direct-to-LDS copies are inline asm that set M0
   themselves: there, M0 is written only by the `s_mov_b32 m0, sN` right
   before each copy, and read by nothing else."""

import os
import re
import shutil
import subprocess

import pytest

from tests.proc import skip_if_gpu_initialised

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "layout_algebra_tiled_amd", "liblt.so")
LLVM = "/opt/rocm/llvm/bin"

_FUNC = re.compile(r"^([0-9a-f]+) <([^>]+)>:$")
_INST = re.compile(r"^\s+(\S+)\s*(.*?)\s*//\s*([0-9A-Fa-f]+):")
_TARGET = re.compile(r"<([^>+]+)\+0x([0-9a-f]+)>")
_VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def _regs(operands: str):
    out = set()
    for a, b, one in _VREG.findall(operands):
        if one:
            out.add(int(one))
        else:
            out.update(range(int(a), int(b) + 1))
    return out


def _functions(text: str):
    """{name: [(addr, mnemonic, operands, comment)]} of a disassembly."""
    funcs, cur = {}, None
    for line in text.splitlines():
        m = _FUNC.match(line)
        if m:
            cur = funcs.setdefault(m.group(2), [])
            continue
        if cur is None:
            continue
        m = _INST.match(line)
        if m:
            comment = line.split("//", 1)[1]
            cur.append((int(m.group(3), 16), m.group(1), m.group(2), comment))
    return funcs


_META = {}


def disasm_meta():
    return _META


@pytest.fixture(scope="module")
def disasm(tmp_path_factory):
    skip_if_gpu_initialised()
    if not os.path.exists(LIB):
        pytest.skip("library not built")
    if not os.path.exists(os.path.join(LLVM, "llvm-objdump")):
        pytest.skip("ROCm llvm-objdump not available")
    d = tmp_path_factory.mktemp("isa")
    lib = d / "liblt.so"
    shutil.copy(LIB, lib)
    subprocess.run([os.path.join(LLVM, "llvm-objdump"), "--offloading", str(lib)], cwd=d, check=True,
                   capture_output=True)
    funcs, addrs = {}, {}
    for co in sorted(d.glob("liblt.so.*gfx950")):
        notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", str(co)],
                               capture_output=True, text=True, check=True).stdout
        for blk in notes.split("  - .agpr_count:")[1:]:
            name = re.search(r"\.name:\s+(\S+)", blk).group(1)
            get = lambda k: int(re.search(k + r":\s+(\d+)", blk).group(1))
            _META[name] = {"spill": get(r"\.vgpr_spill_count") + get(r"\.sgpr_spill_count"),
                           "priv": get(r"\.private_segment_fixed_size")}
        text = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", str(co)],
                              capture_output=True, text=True, check=True).stdout
        for line in text.splitlines():
            m = _FUNC.match(line)
            if m:
                addrs[(co.name, m.group(2))] = int(m.group(1), 16)
        for name, insts in _functions(text).items():
            funcs[(co.name, name)] = insts
    nm = subprocess.run(["nm", "-C", str(LIB)], capture_output=True, text=True, check=True).stdout
    return funcs, addrs, nm


def test_every_tiled_variant_has_device_code_and_a_stub(disasm):
    funcs, _, nm = disasm
    names = {n for (_, n) in funcs}
    want = set()
    for dt in (1, 2):
        for ak in ("0", "1"):
            for bk in ("0", "1"):
                a, b = ("b1" if ak == "1" else "b0"), ("b1" if bk == "1" else "b0")
                # Dp256 (one workgroup per tile, persistent without C),
                # Dp128 (one workgroup per tile, and persistent with and
                # without C) and the split launch of each variant
                # (last template argument: the launch mode)
                t256 = f"_ZN2lt10gemm_tiledILi{dt}ENS_4TCfgILi256ELi256ELi2ELi2ELi64ELi2ELi16EL{a}EL{b}EEE"
                t128 = f"_ZN2lt10gemm_tiledILi{dt}ENS_4TCfgILi256ELi128ELi2ELi2ELi64ELi3ELi16EL{a}EL{b}EEE"
                tsq = f"_ZN2lt10gemm_tiledILi{dt}ENS_4TCfgILi128ELi128ELi2ELi2ELi64ELi4ELi16EL{a}EL{b}EEE"
                tspl = f"_ZN2lt10gemm_tiledILi{dt}ENS_4TCfgILi256ELi256ELi4ELi2ELi64ELi2ELi16EL{a}EL{b}EEE"
                for mode in (0, 2):
                    want.add(t256 + f"Li{mode}EEEvNS_9TiledArgsE")
                for mode in (0, 2, 3):
                    want.add(t128 + f"Li{mode}EEEvNS_9TiledArgsE")
                want.add(tsq + "Li0EEEvNS_9TiledArgsE")   # 128x128: one workgroup per tile
                want.add(tspl + "Li1EEEvNS_9TiledArgsE")
    assert want <= names, sorted(want - names)


_AREG = re.compile(r"\ba\[(\d+):(\d+)\]|\ba(\d+)\b")


def _aregs(operands: str):
    out = set()
    for a, b, one in _AREG.findall(operands):
        if one:
            out.add(int(one))
        else:
            out.update(range(int(a), int(b) + 1))
    return out


def mfma_result_hazards(insts, waits: int = 18):
    """Instructions other than MFMAs that name an MFMA's accumulator
    registers fewer than `waits` wait states after it. An instruction counts
    one, s_nop N counts N+1, and an intervening MFMA counts 4: the SIMD has
    one matrix pipeline, so the next MFMA of the wave issues only when the
    previous one has passed through it (16 cycles for a 16x16x32 MFMA at the
    dense rate; 4 is a safe lower bound). The inline-asm MFMAs are invisible
    to the compiler's hazard recognizer, so this includes any spill or copy
    it places right after one."""
    bad = []
    for i, (_, mn, ops, _) in enumerate(insts):
        if not mn.startswith("v_mfma"):
            continue
        dst = _aregs(ops.split(",")[0])
        ws, j = 0, i + 1
        while j < len(insts) and ws < waits:
            _, mnj, opsj, _ = insts[j]
            if mnj in ("s_branch", "s_endpgm") or mnj.startswith("s_cbranch"):
                break
            if not mnj.startswith("v_mfma") and _aregs(opsj) & dst:
                bad.append((insts[i][:3], insts[j][:3]))
                break
            ws += int(opsj) + 1 if mnj == "s_nop" and opsj.isdigit() else (4 if mnj.startswith("v_mfma") else 1)
            j += 1
    return bad


def test_no_instruction_reads_an_mfma_result_too_early(disasm):
    funcs, _, _ = disasm
    checked = 0
    for key, insts in funcs.items():
        if "gemm_tiled" not in key[1]:
            continue
        bad = mfma_result_hazards(insts)
        assert not bad, f"{key[1]}: {bad[:3]}"
        checked += 1
    assert checked == 56


def test_mfma_hazard_checker_catches_an_early_read():
    frag = """0000000000001000 <k>:
	v_mfma_f32_16x16x32_bf16 a[0:3], v[8:11], v[12:15], a[0:3] // 000000001000: 00000000 00000000
	s_nop 7                                                    // 000000001008: BF800007
	v_accvgpr_read_b32 v0, a1                                  // 00000000100C: 00000000
	s_endpgm                                                   // 000000001010: BF810000
"""
    assert mfma_result_hazards(_functions(frag)["k"])
    def between(n_mfma):
        other = "".join(f"\tv_mfma_f32_16x16x32_bf16 a[{4 * k}:{4 * k + 3}], v[8:11], v[12:15], "
                        f"a[{4 * k}:{4 * k + 3}] // 000000001008: 0\n" for k in range(1, n_mfma + 1))
        return _functions(frag.replace("\ts_nop 7", other + "\ts_nop 7"))["k"]
    # s_nop 7 (8) and two other MFMAs (8) are too few for 18; a third is enough
    assert mfma_result_hazards(between(2))
    assert not mfma_result_hazards(between(3))


def loop_scratch_accesses(insts, base):
    """Scratch (spill) instructions that lie on a cycle of the control-flow
    graph which also issues MFMAs: such a spill or reload repeats every K
    slice. Cycles are the strongly connected components of the
    instruction-level graph (iterative Tarjan)."""
    index_of = {a: i for i, (a, _, _, _) in enumerate(insts)}
    succ = [_successors(insts, i, index_of, base) for i in range(len(insts))]
    n = len(insts)
    index, low, on, stack, comp = [-1] * n, [0] * n, [False] * n, [], [-1] * n
    counter, ncomp = 0, 0
    for root in range(n):
        if index[root] >= 0:
            continue
        work = [(root, 0)]
        while work:
            v, k = work.pop()
            if k == 0:
                index[v] = low[v] = counter
                counter += 1
                stack.append(v)
                on[v] = True
            if k < len(succ[v]):
                work.append((v, k + 1))
                w = succ[v][k]
                if index[w] < 0:
                    work.append((w, 0))
                elif on[w]:
                    low[v] = min(low[v], index[w])
                continue
            if low[v] == index[v]:
                while True:
                    w = stack.pop()
                    on[w] = False
                    comp[w] = ncomp
                    if w == v:
                        break
                ncomp += 1
            if work:
                u = work[-1][0]
                low[u] = min(low[u], low[v])
    members = {}
    for i, c in enumerate(comp):
        members.setdefault(c, []).append(i)
    bad = []
    for c, idx in members.items():
        if len(idx) < 2 or not any(insts[i][1].startswith("v_mfma") for i in idx):
            continue
        bad += [insts[i][:3] for i in idx if insts[i][1].startswith("scratch_")]
    return bad


def test_loop_scratch_checker_finds_a_reload_in_a_loop():
    frag = """0000000000001000 <k>:
	scratch_store_dword off, v0, off                           // 000000001000: 0
	v_mfma_f32_16x16x32_bf16 a[0:3], v[8:11], v[12:15], a[0:3] // 000000001004: 0
	scratch_load_dword v1, off, off                            // 00000000100C: 0
	s_cbranch_scc1 65533                                       // 000000001010: 0 <k+0x4>
	s_endpgm                                                   // 000000001014: 0
"""
    insts = _functions(frag)["k"]
    assert [i[1] for i in loop_scratch_accesses(insts, 0x1000)] == ["scratch_load_dword"]


def test_tiled_kernels_keep_scratch_out_of_the_k_loop(disasm):
    """The tiled kernels keep every value of the K loop in registers: a
    spill there costs a memory round trip per slice. Outside it (index
    set-up, the epilogue) a few dwords may spill. The skinny kernels (A's
    fragments of the slots in flight held in registers) do not spill at all."""
    funcs, addrs, _ = disasm
    meta = disasm_meta()
    tiled = [k for k in funcs if "gemm_tiled" in k[1]]
    assert len(tiled) == 56
    skinny = [k for k in funcs if "gemm_skinny" in k[1]]
    assert len(skinny) == 2
    for key in skinny:
        assert meta[key[1]]["priv"] == 0, (key[1], meta[key[1]])
    for key in tiled:
        assert meta[key[1]]["priv"] <= 16, (key[1], meta[key[1]])
        if meta[key[1]]["priv"]:
            bad = loop_scratch_accesses(funcs[key], addrs[key])
            assert not bad, (key[1], bad[:3])


def _successors(insts, i, index_of, func_addr):
    addr, mn, ops, comment = insts[i]
    if mn == "s_endpgm":
        return []
    nxt = [i + 1] if i + 1 < len(insts) else []
    if mn.startswith("s_branch") or mn.startswith("s_cbranch"):
        m = _TARGET.search(comment)
        assert m, (mn, comment)
        tgt = index_of[func_addr + int(m.group(2), 16)]
        return [tgt] if mn.startswith("s_branch") else nxt + [tgt]
    return nxt


_LGKM = re.compile(r"lgkmcnt\((\d+)\)")


_SPAIR = re.compile(r"^s\[(\d+):(\d+)\]$")
_SREG = re.compile(r"\bs\[(\d+):(\d+)\]|\bs(\d+)\b")


def _sregs(operands: str):
    out = set()
    for a, b, one in _SREG.findall(operands):
        out.update([int(one)] if one else range(int(a), int(b) + 1))
    return out


def _uniform_flags(mn, ops, flags):
    """Track what the structurizer's uniform branch flags make certain:
    SGPR pairs set to -1 or 0 by `s_mov_b64`, and `vcc` certainly zero after
    `s_andn2_b64 vcc, exec, s[a:b]` of a -1 pair or `s_and_b64 vcc, exec,
    s[a:b]` of a 0 pair (zero whatever exec holds), certainly non-zero after
    the opposite pairings (vcc = exec, taken as non-zero: the structurizer
    tests these flags in uniform control flow, where exec is the whole wave). Any other instruction that names a tracked pair's
    registers (or vcc) in any operand forgets that fact, so the tracking only
    ever prunes paths that cannot run. Returns the new frozenset of facts."""
    parts = [x.strip() for x in ops.split(",")] if ops else []
    first = parts[0] if parts else ""
    named = _sregs(ops)
    facts = set()
    for f in flags:   # forget pairs this instruction names
        if f in ("vcc0", "vccN"):
            facts.add(f)
            continue
        lo, hi = (int(x) for x in _SPAIR.match(f[1]).groups())
        if not (named & set(range(lo, hi + 1))) or (mn in ("s_and_b64", "s_andn2_b64") and first == "vcc"):
            facts.add(f)
    if "vcc" in ops and not mn.startswith("s_cbranch_vcc"):
        facts.discard("vcc0")
        facts.discard("vccN")
    if first == "vcc" and len(parts) == 3 and parts[1] == "exec":
        # exec AND NOT -1, exec AND 0: zero whatever exec holds
        if (mn == "s_andn2_b64" and ("m1", parts[2]) in facts) or (mn == "s_and_b64" and ("z", parts[2]) in facts):
            facts.add("vcc0")
        # exec AND -1, exec AND NOT 0: exec itself, non-zero in the uniform
        # control flow where the structurizer tests its flags
        if (mn == "s_and_b64" and ("m1", parts[2]) in facts) or (mn == "s_andn2_b64" and ("z", parts[2]) in facts):
            facts.add("vccN")
    if mn == "s_mov_b64" and _SPAIR.match(first) and len(parts) == 2 and parts[1] in ("-1", "0"):
        facts.add(("m1" if parts[1] == "-1" else "z", first))
    return frozenset(facts)


def _pruned_successors(insts, j, index_of, base, flags):
    """Successors of instruction j, without the branch side that a certainly
    zero vcc rules out."""
    mn = insts[j][1]
    succ = _successors(insts, j, index_of, base)
    if mn in ("s_cbranch_vccz", "s_cbranch_vccnz") and len(succ) == 2:
        if "vcc0" in flags:
            return [succ[1]] if mn == "s_cbranch_vccz" else [succ[0]]
        if "vccN" in flags:
            return [succ[0]] if mn == "s_cbranch_vccz" else [succ[1]]
    return succ


def unwaited_uses(insts, base):
    """(read, instruction) pairs where an instruction names a destination
    register of a transposing read on some path from it before the read is
    retired (or the kernel ends first). Paths that a uniform branch flag
    rules out (`_uniform_flags`) are not followed. Returns (violations,
    number of reads checked)."""
    index_of = {a: i for i, (a, _, _, _) in enumerate(insts)}
    bad, n = [], 0
    for r, (_, mn, ops, _) in enumerate(insts):
        if mn != "ds_read_b64_tr_b16":
            continue
        n += 1
        dest = _regs(ops.split(",")[0])
        # state: (instruction, LDS ops issued since the read (capped), scalar
        # load since, uniform-flag facts)
        seen = set()
        todo = [(j, 0, False, frozenset()) for j in _successors(insts, r, index_of, base)]
        while todo:
            state = todo.pop()
            if state in seen:
                continue
            seen.add(state)
            j, after, smem, flags = state
            _, mnj, opsj, _ = insts[j]
            if mnj == "s_waitcnt":
                m = _LGKM.search(opsj)
                if m and (int(m.group(1)) == 0 or (not smem and after >= int(m.group(1)))):
                    continue
            if _regs(opsj) & dest or mnj == "s_endpgm":
                bad.append((insts[r][:3], insts[j][:3]))
                continue
            after = min(after + (1 if mnj.startswith("ds_") else 0), 64)
            smem = smem or mnj.startswith("s_load") or mnj.startswith("s_buffer_load")
            nflags = _uniform_flags(mnj, opsj, flags)
            todo.extend((k, after, smem, nflags) for k in _pruned_successors(insts, j, index_of, base, nflags))
    return bad, n


def m0_misuse(insts):
    """Instructions that name M0 other than the copies' own `s_mov_b32 m0,
    sN` immediately followed by a direct-to-LDS copy."""
    bad = []
    for i, (_, mn, ops, _) in enumerate(insts):
        if not re.search(r"\bm0\b", ops):
            continue
        ok = (mn == "s_mov_b32" and ops.startswith("m0, s") and i + 1 < len(insts)
              and insts[i + 1][1] == "global_load_lds_dwordx4")
        if not ok:
            bad.append(insts[i][:3])
    return bad


_GOOD = """0000000000001000 <k>:
	ds_read_b64_tr_b16 v[4:5], v0                              // 000000001000: D9C60000 04000000
	ds_read_b64_tr_b16 v[6:7], v0 offset:2048                  // 000000001008: D9C60800 06000000
	v_mfma_f32_16x16x32_bf16 a[0:3], v[8:11], v[12:15], a[0:3]  // 000000001010: 00000000 00000000
	s_cbranch_scc1 2                                           // 000000001018: BF850002 <k+0x24>
	s_waitcnt lgkmcnt(0)                                       // 00000000101C: BF8CC07F
	s_branch 1                                                 // 000000001020: BF820001 <k+0x28>
	s_waitcnt vmcnt(0) lgkmcnt(0)                              // 000000001024: BF8C0070
	v_mov_b32_e32 v8, v4                                       // 000000001028: 7E100304
	s_endpgm                                                   // 00000000102C: BF810000
"""


def test_checker_accepts_waited_reads_and_catches_early_use():
    """The path walk itself, on a hand-written fragment: both paths from the
    reads wait before v4 is copied; moving the copy above the wait, taking
    the wait off one branch path, or waiting with a count that leaves the
    read in flight, must be reported."""
    insts = _functions(_GOOD)["k"]
    assert unwaited_uses(insts, 0x1000) == ([], 2)
    # lgkmcnt(1) after the second read retires the first one only
    partial = _GOOD.replace("s_waitcnt lgkmcnt(0)                                       // 00000000101C",
                            "s_waitcnt lgkmcnt(1)                                       // 00000000101C")
    bad, _ = unwaited_uses(_functions(partial)["k"], 0x1000)
    assert bad and all(b[0][2].startswith("v[6:7]") for b in bad)
    early = _GOOD.replace("v_mfma_f32_16x16x32_bf16 a[0:3], v[8:11]", "v_mfma_f32_16x16x32_bf16 a[0:3], v[4:7]")
    bad, _ = unwaited_uses(_functions(early)["k"], 0x1000)
    assert len(bad) == 2 and all(b[1][1].startswith("v_mfma") for b in bad)
    one_path = _GOOD.replace("s_waitcnt vmcnt(0) lgkmcnt(0)", "s_waitcnt vmcnt(0)")
    bad, _ = unwaited_uses(_functions(one_path)["k"], 0x1000)
    assert {b[1][1] for b in bad} == {"v_mov_b32_e32", "s_endpgm"}   # v4 copied; v6:7 never waited


_FLAGGED = """0000000000001000 <k>:
	ds_read_b64_tr_b16 v[4:5], v0                              // 000000001000: D9C60000 04000000
	s_mov_b64 s[0:1], -1                                       // 000000001008: BE8001C1
	s_andn2_b64 vcc, exec, s[0:1]                              // 00000000100C: 89EA007E
	s_cbranch_vccz 1                                           // 000000001010: BF860001 <k+0x18>
	s_endpgm                                                   // 000000001014: BF810000
	s_waitcnt lgkmcnt(0)                                       // 000000001018: BF8CC07F
	v_mov_b32_e32 v8, v4                                       // 00000000101C: 7E100304
	s_endpgm                                                   // 000000001020: BF810000
"""


def test_checker_follows_only_the_branch_a_uniform_flag_allows():
    """exec AND NOT -1 is zero, so the vccz branch is always taken and the
    early s_endpgm is unreachable; with the flag set to 0, or overwritten
    before the test, or tested as exec AND -1 (vcc = exec, so vccz never
    taken), that s_endpgm is reachable and reported."""
    ok = _functions(_FLAGGED)["k"]
    assert unwaited_uses(ok, 0x1000) == ([], 1)
    zero = _FLAGGED.replace("s_mov_b64 s[0:1], -1 ", "s_mov_b64 s[0:1], 0  ")
    bad, _ = unwaited_uses(_functions(zero)["k"], 0x1000)
    assert [b[1][1] for b in bad] == ["s_endpgm"]
    # a compare that writes the pair forgets what it held
    assert _uniform_flags("v_cmp_gt_u32_e64", "s[0:1], v1, v2", frozenset({("m1", "s[0:1]")})) == frozenset()
    anded = _FLAGGED.replace("s_andn2_b64 vcc, exec, s[0:1]", "s_and_b64 vcc, exec, s[0:1]  ")
    bad, _ = unwaited_uses(_functions(anded)["k"], 0x1000)
    assert [b[1][1] for b in bad] == ["s_endpgm"]


def test_transposing_reads_are_waited_before_use(disasm):
    funcs, addrs, _ = disasm
    kernels, reads = 0, 0
    for key, insts in funcs.items():
        bad, n = unwaited_uses(insts, addrs[key])
        assert not bad, f"{key[1]}: {bad[:3]}"
        if "gemm_tiled" in key[1]:   # the kernels whose copies are inline asm
            assert not m0_misuse(insts), f"{key[1]}: {m0_misuse(insts)[:3]}"
        if n:
            kernels += 1
            reads += n
    # every kernel of a variant with an M/N-major operand issues transposing
    # reads: 3 such variants per dtype, 6 launch configurations each
    assert kernels >= 36 and reads > 1000, (kernels, reads)
