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
