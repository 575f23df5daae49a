"""Static checks on the gfx950 assembly of the attention kernels (no GPU).

The kernels issue their LDS operand reads as inline assembly and wait for
them with explicit ``s_waitcnt lgkmcnt(N)``; the compiler treats such a
read's destination registers as written when the instruction is issued.  If
it copies or spills one of them before the wait (register pressure), the
copy takes the register's old contents.  These tests compile the kernels and
check that this cannot happen: no register spills or scratch use, and no
instruction touches a register of a read still in flight.
"""
import re

import pytest

from comm_fusion_amd import build

_VREG = re.compile(r"^v\[(\d+):(\d+)\]$|^v(\d+)$")
_LGKM = re.compile(r"lgkmcnt\((\d+)\)")


def _vregs(tok: str):
    m = _VREG.match(tok)
    if not m:
        return set()
    if m.group(3) is not None:
        return {int(m.group(3))}
    return set(range(int(m.group(1)), int(m.group(2)) + 1))


def _operands(line: str):
    parts = line.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    return parts[0], [o.strip().split()[0] for o in parts[1].split(",") if o.strip()]


def _kernel_bodies(asm: str, kernel: str = "attn_fwd"):
    """{kernel symbol: [instruction and label lines]} for the kernels whose
    symbol contains `kernel` (default: the attention kernels)."""
    out = {}
    name = None
    for raw in asm.splitlines():
        line = raw.split(";")[0].strip()
        m = re.match(r"^(_Z\S*%s\S*):$" % kernel, line)
        if m:
            name = m.group(1)
            out[name] = []
            continue
        if name is None:
            continue
        if line.startswith(".Lfunc_end"):  # blocks may follow an s_endpgm
            name = None
            continue
        if line and not line.startswith("."):
            out[name].append(line)
        elif re.match(r"^\.LBB\w+:$", line):
            out[name].append(line)
    return out


def _blocks(lines):
    """Basic blocks: (instructions with their line index, successor block ids)."""
    blocks, labels = [], {}
    cur = []
    for i, line in enumerate(lines):
        if line.endswith(":"):
            if cur:
                blocks.append(cur)
                cur = []
            labels[line[:-1]] = len(blocks)
            continue
        cur.append((i, line))
        if line.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
            blocks.append(cur)
            cur = []
    if cur:
        blocks.append(cur)
    # labels that precede an empty run map to the next block
    succ = []
    for k, blk in enumerate(blocks):
        last = blk[-1][1] if blk else ""
        op, ops = _operands(last) if blk else ("", [])
        s = []
        if op.startswith(("s_branch", "s_cbranch")):
            s.append(labels[ops[0]])
        if not op.startswith(("s_branch", "s_endpgm", "s_setpc")) and k + 1 < len(blocks):
            s.append(k + 1)
        succ.append(s)
    return blocks, succ


_MAXPEND = 32


def _merge(a, b):
    """Pending reads after either of two paths: entries aligned from the newest."""
    if a is None:
        return b
    n = max(len(a), len(b))
    pa = [frozenset()] * (n - len(a)) + list(a)
    pb = [frozenset()] * (n - len(b)) + list(b)
    return tuple(x | y for x, y in zip(pa, pb))


def _step(state, line, bad, i):
    op, ops = _operands(line)
    if op.startswith("s_waitcnt"):
        m = _LGKM.search(line)
        if m:
            n = int(m.group(1))
            state = state[len(state) - n:] if n else ()
        return state
    touched = set()
    for o in ops:
        touched |= _vregs(o)
    busy = set().union(*state) if state else set()
    if touched & busy and bad is not None:
        bad.append((i, line))
    if op.startswith(("ds_read", "ds_load")):
        state = state + (frozenset(_vregs(ops[0])),)
    elif op.startswith(("ds_", "s_load", "s_buffer_load")):
        state = state + (frozenset(),)
    return state[-_MAXPEND:]


def early_uses(lines):
    """Instructions that read or write a VGPR of an LDS read not yet waited for.

    LDS reads complete in issue order, so ``lgkmcnt(N)`` leaves the newest N
    outstanding.  Scalar loads share the counter; they are counted in order
    too, which only makes the check stricter.  The reads still in flight are
    propagated over the control-flow graph (branches, fall-through, loop
    back edges) to a fixed point; where paths join, either path's reads
    count as in flight.
    """
    blocks, succ = _blocks(lines)
    inn = [None] * len(blocks)
    inn[0] = ()
    work = [0]
    while work:
        k = work.pop()
        st = inn[k]
        for i, line in blocks[k]:
            st = _step(st, line, None, i)
        for t in succ[k]:
            m = _merge(inn[t], st)
            if m != inn[t]:
                inn[t] = m
                work.append(t)
    bad = []
    for k, blk in enumerate(blocks):
        st = inn[k] if inn[k] is not None else ()
        for i, line in blk:
            st = _step(st, line, bad, i)
    return bad


@pytest.fixture(scope="module")
def asm():
    return build.assembly()


def test_kernels_do_not_spill(asm):
    meta = re.findall(r"\.name:\s+(_Z\S*attn_fwd\S*)|\.(vgpr_spill_count|private_segment_fixed_size):\s+(\d+)",
                      asm)
    assert any(name for name, _, _ in meta), "no attention kernels in the assembly"
    spills = [(k, v) for _, k, v in meta if k and int(v) != 0]
    assert not spills, spills


def test_no_use_of_lds_results_before_their_wait(asm):
    bodies = _kernel_bodies(asm)
    assert len(bodies) >= 4, sorted(bodies)
    for name, lines in bodies.items():
        assert sum(l.startswith("ds_read") for l in lines) > 0, name
        bad = early_uses(lines)
        assert not bad, "%s: %s" % (name, bad[:5])


def test_early_use_checker_catches_a_spill_before_the_wait():
    # the pattern the check exists for: an asm LDS read's destination stored
    # to scratch before its lgkmcnt wait
    lines = ["ds_read_b128 v[96:99], v32 offset:0",
             "scratch_store_dwordx4 off, v[96:99], off offset:140",
             "s_waitcnt lgkmcnt(0)"]
    assert early_uses(lines) == [(1, lines[1])]
    ok = ["ds_read_b128 v[96:99], v32 offset:0",
          "ds_read_b128 v[100:103], v32 offset:1024",
          "s_waitcnt lgkmcnt(1)",
          "v_mfma_f32_32x32x16_bf16 v[0:15], v[96:99], v[200:203], v[0:15]",
          "s_waitcnt lgkmcnt(0)",
          "v_mov_b32_e32 v5, v101"]
    assert early_uses(ok) == []
    # a wait that leaves the read outstanding does not cover it
    late = ["ds_read_b128 v[96:99], v32", "s_waitcnt lgkmcnt(1)", "v_mov_b32_e32 v5, v97"]
    assert early_uses(late) == [(2, late[2])]


# ---- key split: the partial stores are complete before the arrival count ----
#
# In a key-split build every storing wave writes its partial result with
# device-scope (sc1) stores; a workgroup barrier follows, then one thread's
# release add counts the arrival.  The release's own wait only covers the
# stores of that thread's wave, so every wave must wait for its own stores
# (s_waitcnt vmcnt(0)) before it reaches the barrier.

_VM = re.compile(r"vmcnt\((\d+)\)")


def _is_sc1_store(line: str) -> bool:
    op = line.split(None, 1)[0]
    return op.startswith(("global_store", "buffer_store", "flat_store")) and re.search(r"\bsc1\b", line) is not None


def _store_step(pending: bool, line: str, bad, i):
    op = line.split(None, 1)[0]
    if op.startswith("s_waitcnt"):
        m = _VM.search(line)
        if m and int(m.group(1)) == 0:
            return False
        return pending
    if op == "s_barrier" and pending and bad is not None:
        bad.append((i, line))
    if _is_sc1_store(line):
        return True
    return pending


def barriers_with_stores_in_flight(lines):
    """s_barrier instructions reachable while an sc1 store may be outstanding,
    propagated over the control-flow graph (either path's stores count)."""
    blocks, succ = _blocks(lines)
    inn = [None] * len(blocks)
    inn[0] = False
    work = [0]
    while work:
        k = work.pop()
        st = inn[k]
        for i, line in blocks[k]:
            st = _store_step(st, line, None, i)
        for t in succ[k]:
            m = st if inn[t] is None else (inn[t] or st)
            if m != inn[t]:
                inn[t] = m
                work.append(t)
    bad = []
    for k, blk in enumerate(blocks):
        st = bool(inn[k])
        for i, line in blk:
            st = _store_step(st, line, bad, i)
    return bad


def _split_kernels(asm):
    # template argument XS is the first bool: ...Lb1ELb0E (XS = true, TRACE = false)
    return {n: l for n, l in _kernel_bodies(asm).items() if "Lb1ELb0E" in n}


def test_split_partials_complete_before_the_barrier(asm):
    kernels = _split_kernels(asm)
    assert len(kernels) >= 4, sorted(kernels)
    for name, lines in kernels.items():
        stores = [i for i, l in enumerate(lines) if _is_sc1_store(l)]
        adds = [i for i, l in enumerate(lines) if l.startswith("global_atomic_add")]
        assert stores and adds, name
        # the check is not vacuous: between every arrival add and the partial
        # stores laid out before it lies a barrier
        for ad in adds:
            before = [i for i in stores if i < ad]
            assert before and any(l == "s_barrier" for l in lines[before[-1]:ad]), name
        bad = barriers_with_stores_in_flight(lines)
        assert not bad, "%s: %s" % (name, bad[:3])


def test_store_checker_catches_a_barrier_before_the_wait():
    # the ordering this check guards: partial stores, then a barrier whose
    # preceding wait leaves them outstanding, then the release add
    bad = ["global_store_dword v[66:67], v2, off sc1",
           "s_waitcnt vmcnt(63) expcnt(7) lgkmcnt(15)",
           "s_barrier",
           "buffer_wbl2 sc1",
           "s_waitcnt vmcnt(0)",
           "global_atomic_add v1, v1, v66, s[2:3] sc0"]
    assert barriers_with_stores_in_flight(bad) == [(2, "s_barrier")]
    good = bad[:1] + ["s_waitcnt vmcnt(0)"] + bad[1:]
    assert barriers_with_stores_in_flight(good) == []
    # a store on one arm of a branch still counts at the join
    branch = ["s_cbranch_execz .LBB0_2",
              "global_store_dword v[66:67], v2, off sc1",
              ".LBB0_2:",
              "s_barrier"]
    assert barriers_with_stores_in_flight(branch) == [(3, "s_barrier")]
    # plain (non-sc1) stores, such as the epilogue's, are not partials
    assert barriers_with_stores_in_flight(["global_store_dwordx2 v[0:1], v[2:3], off", "s_barrier"]) == []


def _raw_body(asm: str, kernel: str):
    """The listing of the kernel whose symbol contains `kernel`, comments kept."""
    start = re.search(r"^(_Z\S*%s\S*):" % kernel, asm, flags=re.M)
    assert start, kernel
    end = asm.index(".Lfunc_end", start.end())
    return asm[start.end():end].splitlines()


def spill_lanes_in_inner_loops(lines):
    """v_readlane/v_writelane of an SGPR-spill VGPR inside a loop of depth
    >= 2 (in the persistent kernel the k-loops sit inside its tile loop)."""
    spill_regs = set(re.findall(r"implicit-def: \$vgpr(\d+) : SGPR spill to VGPR lane", "\n".join(lines)))
    bad, depth, after_label = [], 0, False
    for raw in lines:
        label = re.match(r"^\.LBB\S+:(.*)", raw.strip())
        if label:
            m = re.search(r"Depth=(\d+)", label.group(1))
            depth, after_label = (int(m.group(1)) if m else 0), True
            continue
        code = raw.split(";")[0].split()
        if not code:
            # a loop header's own depth follows its label on a comment line
            m = re.search(r"Loop Header: Depth=(\d+)", raw)
            if m and after_label:
                depth = max(depth, int(m.group(1)))
            continue
        after_label = False
        if code and code[0] in ("v_readlane_b32", "v_writelane_b32") and depth >= 2:
            if any(r in spill_regs for r in re.findall(r"\bv(\d+)\b", " ".join(code[1:]))):
                bad.append(raw.strip())
    return bad


def test_moe_kernels_do_not_spill():
    a = build.assembly("moe_kernels.hip")
    names = re.findall(r"\.name:\s+(_Z\S*moe\S*)", a)
    assert any("moe_tiles" in n for n in names) and any("moe_persist" in n for n in names), names
    # no kernel uses scratch memory or spills VGPRs; the per-wave-launch
    # kernel spills nothing at all; the persistent one at most a few SGPRs
    # (loop-invariant values of its tile loop) into VGPR lanes that are
    # never touched inside the k-loops
    for key in ("private_segment_fixed_size", "vgpr_spill_count"):
        vals = re.findall(r"\.%s:\s+(\d+)" % key, a)
        assert vals and all(int(v) == 0 for v in vals), (key, vals)
    assert "SGPR spill" not in "\n".join(_raw_body(a, "moe_tiles"))
    persist = _raw_body(a, "moe_persist")
    assert sum("SGPR spill to VGPR lane" in l for l in persist) <= 1
    assert not spill_lanes_in_inner_loops(persist)
    assert max(int(v) for v in re.findall(r"\.sgpr_spill_count:\s+(\d+)", a)) <= 8
    # one workgroup of 8 waves per CU, two waves per SIMD: at most 256 VGPRs
    # per wave and the CU's 160 KiB of LDS
    lds = [int(v) for v in re.findall(r"\.group_segment_fixed_size:\s+(\d+)", a)]
    vg = [int(v) for v in re.findall(r"\.vgpr_count:\s+(\d+)", a)]
    assert max(lds) <= 160 * 1024 and max(vg) <= 256


def test_spill_lane_check_sees_a_spill_in_a_k_loop():
    lines = ["; implicit-def: $vgpr254 : SGPR spill to VGPR lane",
             ".LBB2_6:                  ;   Loop: Header=BB2_6 Depth=1",
             "v_readlane_b32 s4, v254, 0",
             ".LBB2_40:                 ;   Parent Loop BB2_6 Depth=1",
             ";     =>  This Inner Loop Header: Depth=2",
             "v_readlane_b32 s5, v254, 1"]
    # an inner loop's header block: its depth is on the comment line after the label
    assert spill_lanes_in_inner_loops(lines) == ["v_readlane_b32 s5, v254, 1"]
    # a block inside the inner loop
    inner = lines[:3] + [".LBB2_41:                 ;   in Loop: Header=BB2_40 Depth=2", lines[5]]
    assert spill_lanes_in_inner_loops(inner) == ["v_readlane_b32 s5, v254, 1"]
    # outside the inner loops nothing is reported
    assert spill_lanes_in_inner_loops(lines[:3]) == []


# ---- the persistent MoE kernel's hand-off of act rows ----
#
# A Linear-1 tile stores its act rows from every wave (plain stores), each
# wave waits for its own stores (s_waitcnt vmcnt(0)), a workgroup barrier
# follows, then thread 0's device-scope release add (buffer_wbl2, then the
# atomic) counts the tile; Linear-2 tiles of other workgroups read those rows
# once the count is complete.  The release's own wait covers only thread 0's
# wave, so no barrier from which a release add is reached may be passed with
# a store of the wave still in flight.

def _is_store(line: str) -> bool:
    return line.split(None, 1)[0].startswith(("global_store", "buffer_store", "flat_store"))


def _is_release_add(block, j):
    """global_atomic_add at position j of the block with a buffer_wbl2 before
    it in the same block (the compiler's release sequence)."""
    op = block[j][1].split(None, 1)[0]
    return op.startswith("global_atomic_add") and any(l.startswith("buffer_wbl2") for _, l in block[:j])


def barriers_before_a_release_with_stores_in_flight(lines):
    blocks, succ = _blocks(lines)
    n = len(blocks)
    # forward: a store of this wave may be outstanding (no vmcnt(0) since)
    inn = [None] * n
    inn[0] = False
    work = [0]

    def step(st, line):
        op = line.split(None, 1)[0]
        if op.startswith("s_waitcnt"):
            m = _VM.search(line)
            return False if (m and int(m.group(1)) == 0) else st
        return True if _is_store(line) else st
    while work:
        k = work.pop()
        st = inn[k]
        for _, line in blocks[k]:
            st = step(st, line)
        for t in succ[k]:
            m = st if inn[t] is None else (inn[t] or st)
            if m != inn[t]:
                inn[t] = m
                work.append(t)
    # backward: from the start of a block, a release add is reached before
    # any barrier on some path
    reach = [False] * n
    changed = True
    while changed:
        changed = False
        for k in range(n):
            v = None
            for j, (_, line) in enumerate(blocks[k]):
                if _is_release_add(blocks[k], j):
                    v = True
                    break
                if line.startswith("s_barrier"):
                    v = False
                    break
            if v is None:
                v = any(reach[t] for t in succ[k])
            if v and not reach[k]:
                reach[k] = changed = True
    bad = []
    for k in range(n):
        st = bool(inn[k])
        for j, (i, line) in enumerate(blocks[k]):
            if line.startswith("s_barrier") and st:
                lead = None
                for jj in range(j + 1, len(blocks[k])):
                    if _is_release_add(blocks[k], jj):
                        lead = True
                        break
                    if blocks[k][jj][1].startswith("s_barrier"):
                        lead = False
                        break
                if lead is None:
                    lead = any(reach[t] for t in succ[k])
                if lead:
                    bad.append((i, line))
            st = step(st, line)
    return bad


def test_persistent_moe_counts_a_tile_only_after_every_wave_stored_it():
    bodies = {n: l for n, l in _kernel_bodies(build.assembly("moe_kernels.hip"), "moe_persist").items()}
    assert len(bodies) == 1
    for name, lines in bodies.items():
        blocks, _ = _blocks(lines)
        releases = [(k, j) for k, b in enumerate(blocks) for j in range(len(b)) if _is_release_add(b, j)]
        assert releases, "no release add found in " + name
        assert not barriers_before_a_release_with_stores_in_flight(lines)


def test_release_checker_catches_a_barrier_before_the_stores_complete():
    bad = ["global_store_dwordx2 v[0:1], v[2:3], off",
           "s_waitcnt vmcnt(63) expcnt(7) lgkmcnt(15)",
           "s_barrier",
           "buffer_wbl2 sc1",
           "s_waitcnt vmcnt(0)",
           "global_atomic_add v1, v1, v66, s[2:3] sc1"]
    assert barriers_before_a_release_with_stores_in_flight(bad) == [(2, "s_barrier")]
    good = bad[:1] + ["s_waitcnt vmcnt(0)"] + bad[1:]
    assert barriers_before_a_release_with_stores_in_flight(good) == []
    # stores before a barrier that leads to no release (the Linear-2
    # epilogue's Combine stores before the next tile's barrier) are fine
    other = ["global_store_dwordx4 v[0:1], v[2:5], off", "s_barrier", "global_atomic_add v1, v1, v66, s[2:3]"]
    assert barriers_before_a_release_with_stores_in_flight(other) == []


def test_moe_lds_results_not_used_before_their_wait():
    # the MoE kernel reads its MFMA operands with the same explicit LDS reads
    bodies = {n: l for n, l in _kernel_bodies(build.assembly("moe_kernels.hip"), "moe_").items()
              if "moe_tiles" in n or "moe_persist" in n}
    assert len(bodies) == 2, sorted(bodies)
    for name, lines in bodies.items():
        assert sum(l.startswith("ds_read_b128") for l in lines) >= 48, name
        bad = early_uses(lines)
        assert not bad, "%s: %s" % (name, bad[:5])


def test_persistent_moe_reads_act_at_device_scope():
    # the Linear-2 tiles of the persistent kernel copy act rows written by
    # other workgroups of the same launch: those copies carry sc1 (read past
    # the XCD's L2); the per-wave kernel reads act after a launch boundary
    a = build.assembly("moe_kernels.hip")
    persist = "\n".join(_raw_body(a, "moe_persist"))
    tiles = "\n".join(_raw_body(a, "moe_tiles"))
    lds_copies = re.compile(r"^\s*buffer_load_dwordx4\b.*\blds\b.*$", re.M)
    p_sc1 = [l for l in lds_copies.findall(persist) if re.search(r"\bsc1\b", l)]
    assert p_sc1, "no device-scope act copies in moe_persist"
    assert not [l for l in lds_copies.findall(tiles) if re.search(r"\bsc1\b", l)]
    # thread 0's acquire after it observes the count (pairs with the release)
    assert re.search(r"^\s*buffer_inv sc1\b", persist, re.M)


# ---- d = 64: the issue priority is raised only for a slot's softmax slice ----
#
# At d = 64 each steady-loop slot raises the wave's issue priority
# (s_setprio 1) for its VALU slice and drops it (s_setprio 0) before the next
# slot's MFMA.  Check over the control-flow graph that no s_barrier,
# s_endpgm or MFMA is reached while the priority may still be raised, and
# that only the d = 64 kernels change it.

_PRIO = re.compile(r"^s_setprio\s+(\S+)")


def _prio_step(raised: bool, line: str, bad, i):
    m = _PRIO.match(line)
    if m:
        return int(m.group(1), 0) != 0
    if raised and bad is not None and line.startswith(("s_barrier", "s_endpgm", "v_mfma")):
        bad.append((i, line))
    return raised


def raised_priority_reaches(lines):
    """Barriers, program ends and MFMAs reachable with the priority raised."""
    blocks, succ = _blocks(lines)
    inn = [None] * len(blocks)
    inn[0] = False
    work = [0]
    while work:
        k = work.pop()
        st = inn[k]
        for i, line in blocks[k]:
            st = _prio_step(st, line, None, i)
        for t in succ[k]:
            m = st if inn[t] is None else (inn[t] or st)
            if m != inn[t]:
                inn[t] = m
                work.append(t)
    bad = []
    for k, blk in enumerate(blocks):
        st = bool(inn[k])
        for i, line in blk:
            st = _prio_step(st, line, bad, i)
    return bad


def test_d64_priority_covers_only_the_softmax_slices(asm):
    bodies = _kernel_bodies(asm)
    d64 = {n: l for n, l in bodies.items() if "attn_fwdILi64E" in n}
    d128 = {n: l for n, l in bodies.items() if "attn_fwdILi128E" in n}
    assert d64 and d128
    for name, lines in d64.items():
        raises = [l for l in lines if _PRIO.match(l) and int(_PRIO.match(l).group(1), 0) != 0]
        # one raise per steady-loop slot: as many as the loop has MFMAs, at least
        assert len(raises) >= 16, name
        bad = raised_priority_reaches(lines)
        assert not bad, "%s: %s" % (name, bad[:3])
    for name, lines in d128.items():
        assert not [l for l in lines if _PRIO.match(l)], name


def test_priority_checker_catches_a_raise_held_into_a_barrier():
    ok = ["s_setprio 1", "v_exp_f32_e32 v1, v1", "s_setprio 0",
          "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]", "s_barrier", "s_endpgm"]
    assert raised_priority_reaches(ok) == []
    # the drop sits on one path only: the other reaches the barrier raised
    bad = ["s_setprio 1", "v_exp_f32_e32 v1, v1", "s_cbranch_scc1 .LBB0_2",
           "s_setprio 0", ".LBB0_2:", "s_barrier", "s_endpgm"]
    assert raised_priority_reaches(bad) == [(5, "s_barrier"), (6, "s_endpgm")]
    # an MFMA issued before the drop
    late = ["s_setprio 1", "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]", "s_setprio 0"]
    assert raised_priority_reaches(late) == [(1, late[1])]
