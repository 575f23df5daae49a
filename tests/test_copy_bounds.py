"""Host-side bounds check of the attention kernel's global reads (no GPU).

The K/V tile copies address their source as a wave-uniform base plus a
32-bit per-lane byte offset, and rows past the sequence end (the ragged last
tile) are clamped to the last row inside it.  A first version of this
addressing applied the clamp as an unsigned offset and, for a copy whose
whole 16-row slab lay past the end, wrapped to read ~4 GB past the buffer.
This test restates the documented copy addressing (which 1 KiB copies each
wave issues, which row and 16-byte chunk each lane fetches, the per-lane
offsets in 32-bit arithmetic, the clamp on the row index, the key range of
every key group and key-split part) and checks, for every launch shape the
kernel is built in, every shape the GPU tests run and the five workloads, at
both row strides (Hl*d for [B][S][Hl][d] inputs, H*d for the
sequence-partitioned inputs read in place), that every 16-byte read of K, V
and Q lies inside its tensor.  A mutant that restores a slab-wide unsigned
shift as the clamp is shown to read out of bounds.
"""
import os
import sys

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

import test_gpu_key_split as gks  # noqa: E402  (shape tables only)
import test_gpu_parity as gpar  # noqa: E402
import test_gpu_sweep as gsw  # noqa: E402
from ua_inputs import WORKLOADS  # noqa: E402

U32 = 1 << 32

# Every instantiation of the attention kernel: (d, waves, row blocks per
# wave, keys per tile, key groups).  The split (XS) builds exist for the
# 8-wave shapes only.
INSTANCES = [
    (128, 8, 1, 64, 1), (128, 4, 1, 64, 1), (128, 8, 1, 32, 2),
    (64, 8, 2, 32, 1), (64, 8, 1, 64, 1), (64, 4, 1, 64, 1), (64, 8, 1, 32, 2),
]
MAX_SPLIT = 4
MIN_SPLIT_UNITS = 8


def group_keys(S, KB, KS, grp, split, n_split, xs):
    """(first key, tiles, keys) of one key group of one workgroup."""
    nt_all = -(-S // KB)
    if xs:
        U = nt_all // KS
        u0, u1 = split * U // n_split, (split + 1) * U // n_split
        ntiles = u1 - u0
        kvbase = (u0 * KS + grp * ntiles) * KB
    else:
        ntiles = nt_all // KS
        kvbase = grp * ntiles * KB
    skv = min(S - kvbase, ntiles * KB)
    return kvbase, ntiles, skv


def copy_reads(S, rs, D, NW, KB, KS, grp, split, n_split, xs, clamp="row"):
    """Byte offsets (relative to the head's first element) of every 16-byte
    read the key group's waves issue for K and for V, over all its tiles."""
    TILE = KB * D * 2
    NCP = TILE // 1024
    NWG = NW // KS
    SPLIT = NCP < NWG
    NLD = 1 if SPLIT else NCP // NWG
    CPG = KB // 16
    kvbase, ntiles, skv = group_keys(S, KB, KS, grp, split, n_split, xs)
    lane = np.arange(64, dtype=np.int64)
    lrow = lane >> 2
    k_chunk = ((lane & 3) ^ ((lane >> 4) & 3)) * 16
    v_chunk = (lane & 3) * 16
    kv0 = np.arange(ntiles, dtype=np.int64)[:, None] * KB       # tiles x 1
    out = {"k": [], "v": []}
    for wq in range(NWG):
        kcp0 = wq if SPLIT else wq * NLD
        vcp0 = wq - NCP if SPLIT else wq * NLD
        kcopies = (not SPLIT) or wq < NCP
        vcopies = (not SPLIT) or (NCP <= wq < 2 * NCP)
        for name, copies, cp0, chunk in (("k", kcopies, kcp0, k_chunk), ("v", vcopies, vcp0, v_chunk)):
            if not copies:
                continue
            for n in range(NLD):
                cp = cp0 + n
                row = 16 * (cp % CPG) + lrow                       # lanes
                col = (cp // CPG) * 32
                full = ((row * rs + col) * 2 + chunk) % U32        # precomputed per-lane offset
                last = skv - 1 - kv0                               # tiles x 1
                partial = kv0 + KB > skv
                if clamp == "row":
                    r = np.minimum(row[None, :], last)
                    o = ((r * rs + col) * 2 + chunk[None, :]) % U32
                else:
                    # mutant: shift the whole 16-row slab back, as an unsigned offset
                    shift = np.maximum(0, 16 * (cp % CPG) + 15 - last)
                    o = (full[None, :] - shift * rs * 2) % U32
                o = np.where(partial, o, full[None, :])
                out[name].append(2 * (kvbase + kv0) * rs + o)      # source base + lane offset
    return {k: np.concatenate(v, axis=None) if v else np.zeros(0, np.int64) for k, v in out.items()}


def q_reads(S, rs, D, NW, RB, KS, n_qtiles):
    """Byte offsets of the Q loads of every query tile (relative to the head)."""
    NWG = NW // KS
    BR = 32 * RB * NWG
    lane = np.arange(64, dtype=np.int64)
    il, g = lane & 31, lane >> 5
    qt = np.arange(n_qtiles, dtype=np.int64)[:, None, None]
    wq = np.arange(NWG, dtype=np.int64)[None, :, None]
    offs = []
    for rb in range(RB):
        s_q = qt * BR + wq * 32 * RB + rb * 32 + il
        s_ld = np.minimum(s_q, S - 1)
        for kk in range(D // 16):
            offs.append(2 * (s_ld * rs + 16 * kk + 8 * g))
    return np.concatenate(offs, axis=None)


def plans(S, inst):
    """(xs, n_split) pairs the instantiation can run for this S."""
    d, NW, RB, KB, KS = inst
    nt_all = -(-S // KB)
    if KS == 2 and (nt_all < 2 or nt_all % 2):
        return []                        # key groups only run for an even tile count
    out = [(False, 1)]
    if NW == 8:
        U = nt_all // KS
        for n in range(1, MAX_SPLIT + 1):
            if n == 1 or U // n >= MIN_SPLIT_UNITS:
                out.append((True, n))
    return out


def check_shape(B, S, H, P, rank, d, clamp="row"):
    """Out-of-range reads (tensor, count) over every launch the shape can run."""
    Hl = H // P
    bad = []
    for inst in INSTANCES:
        if inst[0] != d:
            continue
        _, NW, RB, KB, KS = inst
        BR = 32 * RB * NW // KS
        n_qtiles = -(-S // BR)
        for in_heads, in_head0s in ((Hl, [0]), (H, sorted({rank * Hl, (P - 1) * Hl}))):
            rs = in_heads * d
            nbytes = B * S * in_heads * d * 2
            heads = [(b * S * in_heads + h0 + h) * d * 2
                     for b in sorted({0, B - 1}) for h0 in in_head0s for h in sorted({0, Hl - 1})]
            qr = q_reads(S, rs, d, NW, RB, KS, n_qtiles)
            for hb in heads:
                if (hb + qr).min() < 0 or (hb + qr).max() + 16 > nbytes:
                    bad.append(("q", inst, in_heads))
            for xs, n in plans(S, inst):
                for split in range(n):
                    for grp in range(KS):
                        rd = copy_reads(S, rs, d, NW, KB, KS, grp, split, n, xs, clamp)
                        for name, offs in rd.items():
                            if offs.size == 0:
                                continue
                            lo, hi = offs.min(), offs.max()
                            for hb in heads:
                                if hb + lo < 0 or hb + hi + 16 > nbytes:
                                    bad.append((name, inst, in_heads, xs, n, split, grp))
    return bad


def _gpu_shapes():
    shapes = {tuple(c[:6]) for c in gpar.SMALL}
    shapes |= {tuple(c[:6]) for c in gpar.IO_CASES}
    shapes |= {tuple(c[:6]) for c in gsw.SHAPES + gsw.SHAPES_B + gsw.SHAPES_SPLIT}
    shapes |= {tuple(c[:6]) for c in gks.SPLIT_CASES}
    # the edge-case tests' shapes (tiny sequences with many heads, long
    # sequences with one local head, running-max patterns)
    shapes |= {(1, 1, 128, 1, 0, 64), (1, 2, 256, 2, 0, 64), (1, 33, 272, 1, 0, 64),
               (1, 1, 128, 1, 0, 128), (1, 2, 256, 2, 1, 128),
               (1, 524290, 2, 2, 1, 64), (1, 262150, 2, 2, 0, 128),
               (1, 1030, 64, 1, 0, 128), (1, 1030, 4, 1, 0, 64), (1, 1024, 4, 1, 0, 128), (1, 1024, 4, 1, 0, 64)}
    return sorted(shapes)


GPU_SHAPES = _gpu_shapes()


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_workload_reads_stay_inside_their_tensors(name):
    w = WORKLOADS[name]
    assert check_shape(w.B, w.S, w.H, w.P, w.rank, w.d) == []


def test_gpu_test_shapes_read_inside_their_tensors():
    assert len(GPU_SHAPES) > 60
    bad = {s: check_shape(*s) for s in GPU_SHAPES}
    bad = {s: b[:3] for s, b in bad.items() if b}
    assert not bad, bad


def test_every_copy_lane_fetches_each_tile_byte_once():
    # the addressing being bounds-checked is the real one: over a full tile
    # the copies of a key group fetch every 16-byte chunk of the tile's K
    # (and V) rows exactly once
    for d, NW, RB, KB, KS in INSTANCES:
        rs = 3 * d                      # an arbitrary row stride wider than d
        rd = copy_reads(4 * KB, rs, d, NW, KB, KS, 0, 0, 1, False)
        for name in ("k", "v"):
            first = rd[name][rd[name] < KB * rs * 2]            # tile 0
            rows, within = np.divmod(first, rs * 2)
            assert np.all(within < d * 2)
            assert len(first) == KB * d * 2 // 16
            assert len(np.unique(first)) == len(first)


def test_unsigned_slab_clamp_mutant_reads_out_of_bounds():
    # 200 keys: the last 64-key tile holds 8, so three of its four 16-row
    # slabs lie wholly past the end; shifting a slab back by an unsigned
    # offset wraps for those lanes
    assert check_shape(2, 200, 8, 8, 3, 128) == []
    bad = check_shape(2, 200, 8, 8, 3, 128, clamp="slab")
    assert bad and {b[0] for b in bad} <= {"k", "v"}
