"""The MoE calls of the C-ABI library (CPU only): every function
include/moe_combine.h declares is exported; arguments are validated on the
host before any device access; this rank's receive layout matches the
oracle's slot list; and the documented dealing of tiles over a launch's
blocks covers every tile of both kinds exactly once."""
import ctypes
import os
import re

import numpy as np
import pytest

import comm_fusion_amd as ua
import oracle.moe_oracle as mo
from comm_fusion_amd._moe_binding import MoeShape, _lib
from moe_inputs import MOE_WORKLOADS, MoeWorkload, moe_tensors

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_combine.h")
A = 0x10000  # aligned fake device addresses: every call below fails validation first


def test_exports_every_declared_function():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = set(re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", text, flags=re.M))
    assert names >= {"moe_recv_layout", "moe_experts_combine", "moe_experts_local", "moe_combine_scatter"}
    L = ctypes.CDLL(ua.lib_path())
    for n in names:
        assert hasattr(L, n), n
    assert re.search(r"MOE_EXPERT_WAVE\s*=\s*0", text) and re.search(r"MOE_INTERLEAVED\s*=\s*1", text)
    assert re.search(r"#define\s+MOE_MAX_WAVE\s+32\b", text)


def _combine(shp, off, P=2, schedule=1, G=4, x=A, rs=A, w=A, W1=A, W2=A, out=A, act=A):
    o = np.asarray(off, np.int64)
    return _lib().moe_experts_combine(x, rs, w, o.ctypes.data if o.size else None, W1, W2, P,
                                      ctypes.byref(shp) if shp is not None else None, out, act, schedule, G, None)


def test_experts_call_validation():
    ok = MoeShape(64, 256, 128, 8, 2)      # T, hidden, inter, E, k
    off = [0, 3, 3, 10, 12]                # E/P = 4 local experts (P = 2)
    assert _combine(None, off) == ua.UA_ERR_NULL
    assert _combine(MoeShape(64, 384, 128, 8, 2), off) == ua.UA_ERR_SHAPE      # hidden % 256
    assert _combine(MoeShape(64, 256, 192, 8, 2), off) == ua.UA_ERR_SHAPE      # inter % 128
    assert _combine(MoeShape(64, 256, 128, 7, 2), off) == ua.UA_ERR_SHAPE      # E % P
    assert _combine(MoeShape(64, 256, 128, 8, 9), off) == ua.UA_ERR_SHAPE      # k > E
    assert _combine(ok, off, schedule=2) == ua.UA_ERR_UNSUPPORTED
    assert _combine(ok, off, G=0) == ua.UA_ERR_UNSUPPORTED
    assert _combine(ok, off, G=33) == ua.UA_ERR_UNSUPPORTED
    assert _combine(ok, [1, 3, 3, 10, 12]) == ua.UA_ERR_SHAPE                 # offsets[0] != 0
    assert _combine(ok, [0, 3, 2, 10, 12]) == ua.UA_ERR_SHAPE                 # decreasing
    assert _combine(ok, [0, 3, 3, 10, 2 * 64 * 2 + 1]) == ua.UA_ERR_SHAPE      # N > P*T*k
    assert _combine(ok, [0, 0, 0, 0, 0], x=0, rs=0, w=0, W1=0, W2=0, out=0, act=0) == ua.UA_OK  # empty
    assert _combine(ok, off, act=0) == ua.UA_ERR_NULL
    assert _combine(ok, off, out=A + 8) == ua.UA_ERR_ALIGN
    # 32-bit offsets: one expert's W1 must span fewer than 2^32 bytes
    assert _combine(MoeShape(64, 1 << 16, 1 << 14, 8, 2), off) == ua.UA_ERR_UNSUPPORTED
    L = _lib()
    assert L.moe_experts_local(A, A, A, np.asarray(off, np.int64).ctypes.data, A, A, 2, ctypes.byref(ok),
                               A, A, 0, None) == ua.UA_ERR_UNSUPPORTED
    assert L.moe_combine_scatter(A, A, -1, 2, ctypes.byref(ok), A, None) == ua.UA_ERR_SHAPE
    assert L.moe_combine_scatter(0, 0, 0, 2, ctypes.byref(ok), 0, None) == ua.UA_OK
    assert L.moe_combine_scatter(A, A, 5, 2, ctypes.byref(ok), A + 4, None) == ua.UA_ERR_ALIGN


@pytest.mark.parametrize("name", ["moe_tiny", "moe_small", "moe_small_skewed"])
def test_recv_layout_matches_the_oracle_slots(name):
    w = MOE_WORKLOADS[name]
    _, idx, _, _, _ = moe_tensors(w)
    for r in range(w.P):
        off, slots = ua.moe_recv_layout(idx, r, w.P, w.hidden, w.inter, w.E)
        ref = mo.rank_slots(idx, r, w.P, w.E)
        assert off[0] == 0 and off[-1] == len(ref) == len(slots)
        np.testing.assert_array_equal(np.diff(off), np.bincount(ref[:, 0], minlength=w.E_l))
        np.testing.assert_array_equal(slots, (ref[:, 1] * w.T + ref[:, 2]) * w.k + ref[:, 3])


def test_recv_layout_rejects_bad_expert_ids_and_small_capacity():
    w = MoeWorkload("t", P=2, rank=0, T=4, hidden=256, inter=128, E=4, k=2, seed=1)
    _, idx, _, _, _ = moe_tensors(w)
    bad = idx.copy()
    bad[1, 2, 1] = 4
    with pytest.raises(ua.UAError):
        ua.moe_recv_layout(bad, 0, 2, 256, 128, 4)
    shp = MoeShape(4, 256, 128, 4, 2)
    off = np.zeros(3, np.int64)
    slots = np.zeros(1, np.int32)
    st = _lib().moe_recv_layout(idx.ctypes.data, 0, 2, ctypes.byref(shp), off.ctypes.data, slots.ctypes.data, 1)
    assert st == ua.UA_ERR_SHAPE
    assert _lib().moe_recv_layout(idx.ctypes.data, 2, 2, ctypes.byref(shp), off.ctypes.data,
                                  slots.ctypes.data, 16) == ua.UA_ERR_RANK


# ---- the dealing of tiles over blocks (restated from the kernel's rule) ----

def _deal(n_l1, n_l2):
    """Block b of a launch is a Linear-2 tile when floor((b+1) n_l2 / N) >
    floor(b n_l2 / N); its index among its kind's tiles follows."""
    N = n_l1 + n_l2
    out = []
    for b in range(N):
        c2, c2n = b * n_l2 // N, (b + 1) * n_l2 // N
        out.append((1, c2) if c2n > c2 else (0, b - c2))
    return out


@pytest.mark.parametrize("n_l1,n_l2", [(0, 7), (9, 0), (512, 896), (896, 512), (1, 1000), (1000, 1), (37, 53)])
def test_every_tile_is_dealt_once_and_kinds_interleave(n_l1, n_l2):
    d = _deal(n_l1, n_l2)
    assert sorted(i for k, i in d if k == 0) == list(range(n_l1))
    assert sorted(i for k, i in d if k == 1) == list(range(n_l2))
    if n_l1 and n_l2:
        # in every stretch of blocks the share of Linear-2 tiles stays within
        # one tile of n_l2 / N
        N = n_l1 + n_l2
        kinds = np.array([k for k, _ in d])
        c = np.concatenate([[0], np.cumsum(kinds)])
        b = np.arange(N + 1)
        assert np.all(np.abs(c - b * n_l2 / N) < 1.0)


# ---- the persistent form's queue (restated from the launch and the kernel) ----

MAX_WAVE = 32


def _queue(n_e, G, interleaved, BM=256, l1_cols=16, l2_cols=28):
    """Every queue position of every launch, decoded as the kernel does:
    launches of whole waves of at most 32 experts; per launch, phases
    (Expert-Wave: L1 w, L2 w, ...; interleaved: L1 w0, L2 w-1 + L1 w, ...,
    L2 last), each phase dealt like a launch of the per-wave form.  Returns
    [(launch, position, kind, expert, token tile, feature tile)]."""
    E_l = len(n_e)
    mt = [-(-int(n) // BM) for n in n_e]
    n_waves = -(-E_l // G)
    per_launch = MAX_WAVE // G
    out = []
    for q, w0 in enumerate(range(0, n_waves, per_launch)):
        w1 = min(n_waves, w0 + per_launch)
        phases = []

        def phase(l1w, l2w):
            segs = []
            cnt = [0, 0]
            for kind, w in ((1, l2w), (0, l1w)):
                if w < 0:
                    continue
                for e in range(w * G, min((w + 1) * G, E_l)):
                    if n_e[e] == 0:
                        continue
                    nt = l1_cols if kind == 0 else l2_cols
                    segs.append((kind, e, cnt[kind], mt[e], nt))
                    cnt[kind] += mt[e] * nt
            if cnt[0] + cnt[1]:
                phases.append((segs, cnt[0], cnt[1]))
        if interleaved:
            phase(w0, -1)
            for w in range(w0 + 1, w1):
                phase(w, w - 1)
            phase(-1, w1 - 1)
        else:
            for w in range(w0, w1):
                phase(w, -1)
                phase(-1, w)
        pos = 0
        for segs, n1, n2 in phases:
            N = n1 + n2
            for b in range(N):
                c2, c2n = b * n2 // N, (b + 1) * n2 // N
                kind, idx = (1, c2) if c2n > c2 else (0, b - c2)
                hit = [s for s in segs if s[0] == kind and s[2] <= idx < s[2] + s[3] * s[4]]
                assert len(hit) == 1
                _, e, t0, m_t, _ = hit[0]
                nn, mm = divmod(idx - t0, m_t)
                out.append((q, pos + b, kind, e, mm, nn))
            pos += N
    return out


@pytest.mark.parametrize("G", [1, 3, 8, 32])
@pytest.mark.parametrize("interleaved", [True, False])
@pytest.mark.parametrize("n_e", [[455, 545, 0, 1, 256, 257, 512, 30] * 4, [600] * 70, [0, 0, 5]])
def test_persistent_queue_deals_every_tile_once_after_its_dependencies(G, interleaved, n_e):
    q = _queue(n_e, G, interleaved)
    tiles = [(k, e, mm, nn) for _, _, k, e, mm, nn in q]
    want = [(k, e, mm, nn) for e, n in enumerate(n_e) for mm in range(-(-n // 256))
            for k, ncol in ((0, 16), (1, 28)) for nn in range(ncol)]
    assert sorted(tiles) == sorted(want)
    # a Linear-2 tile's 16 Linear-1 tiles come earlier in the same launch's
    # queue (so the workgroups that took them are running and never wait)
    where = {(k, e, mm, nn): (launch, pos) for launch, pos, k, e, mm, nn in q}
    for launch, pos, k, e, mm, nn in q:
        if k == 1:
            for c in range(16):
                lq, lp = where[(0, e, mm, c)]
                assert lq == launch and lp < pos
    # interleaved: in every launch but the first wave's, a phase holds both kinds
    if interleaved and G < len(n_e):
        kinds = {}
        for launch, pos, k, *_ in q:
            kinds.setdefault(launch, set()).add(k)
        assert all(v == {0, 1} for v in kinds.values())


def test_persistent_queue_catches_a_reversed_phase_order():
    # a mutant that runs each wave's Linear-2 phase before its Linear-1 phase
    # puts Linear-2 tiles ahead of their dependencies
    q = _queue([300, 40], 1, False)
    order = sorted(q, key=lambda r: (r[0], r[2] == 0, r[1]))  # kind 1 first
    seen = set()
    bad = False
    for _, _, k, e, mm, nn in order:
        if k == 1 and any((0, e, mm, c) not in seen for c in range(16)):
            bad = True
        seen.add((k, e, mm, nn))
    assert bad


def test_persistent_workspace_size_and_validation():
    ok = MoeShape(64, 256, 128, 8, 2)
    n = _lib().moe_workspace_bytes(2, ctypes.byref(ok))
    # header of 64 words (a queue counter per launch, the timeout count) plus
    # one word per token tile: N <= 2*64*2 = 256 rows over 4 local experts
    # give at most 1 + 4 token tiles
    assert n % 256 == 0 and n >= 4 * (64 + 5)
    assert _lib().moe_workspace_bytes(2, ctypes.byref(MoeShape(64, 384, 128, 8, 2))) == 0
    off = np.asarray([0, 3, 3, 10, 12], np.int64)
    L = _lib()

    def call(ws, nbytes, G=4):
        return L.moe_experts_combine_ws(A, A, A, off.ctypes.data, A, A, 2, ctypes.byref(ok), A, A, 1, G, ws, nbytes,
                                        None)
    assert call(None, n) == ua.UA_ERR_NULL
    assert call(A + 4, n) == ua.UA_ERR_ALIGN
    assert call(A, 4 * 64) == ua.UA_ERR_WORKSPACE          # no room for the 4 token tiles
    assert call(A, n, G=0) == ua.UA_ERR_UNSUPPORTED
    assert L.moe_experts_local_ws(A, A, A, off.ctypes.data, A, A, 2, ctypes.byref(ok), A, A, 4, None, n,
                                  None) == ua.UA_ERR_NULL
    zero = np.zeros(5, np.int64)
    assert L.moe_experts_combine_ws(0, 0, 0, zero.ctypes.data, 0, 0, 2, ctypes.byref(ok), 0, 0, 1, 4, None, 0,
                                    None) == ua.UA_OK  # empty
    # more than 32 launches: 1056 local experts at one per wave
    big = MoeShape(1, 256, 128, 1056, 1)
    boff = np.zeros(1057, np.int64)
    boff[-1] = 1
    assert L.moe_experts_combine_ws(A, A, A, boff.ctypes.data, A, A, 1, ctypes.byref(big), A, A, 1, 1, A, 1 << 20,
                                    None) == ua.UA_ERR_UNSUPPORTED
