"""Host-side check of the key-split launches' index arithmetic (no GPU).

Restates, from the kernel's documented rules, which keys each split workgroup
and key group processes and where it writes its partial results, for every
shape the GPU tests split plus the two DiT workloads, and checks that every
K/V tile of a query tile is processed exactly once and that every partial
and count index lies inside the bytes ua_workspace_bytes reports.
"""
import numpy as np
import pytest

import comm_fusion_amd as ua

SHAPES = [
    # B, S, H, d, P
    (1, 4096, 24, 128, 8), (1, 16384, 24, 128, 8), (1, 8176, 8, 128, 8), (2, 2048, 8, 64, 2),
    (1, 8192, 40, 64, 8), (1, 16384, 48, 64, 8), (1, 3584, 8, 64, 8), (1, 4064, 8, 128, 8),
    (1, 8192, 8, 128, 8), (1, 4096, 16, 128, 8), (1, 16384, 40, 128, 8), (1, 32768, 40, 128, 8),
]


def _plan_shape(B, S, Hl, d, n):
    """The two candidate shapes of a split launch, as (waves, row blocks, keys
    per tile, key groups): the plain call's shape (the documented launch-shape
    rule) and the 8-wave 256-row shape on 64-key tiles."""
    if B * Hl * -(-S // 256) < 128:
        nt = -(-S // 32)
        plain = (8, 1, 32, 2) if nt >= 2 and nt % 2 == 0 else (4, 1, 64, 1)
    elif d == 64 and B * Hl * -(-S // 512) >= 128 and \
            -(-B * Hl * -(-S // 512) // 256) * min(S, 512) * 24 <= -(-B * Hl * -(-S // 256) // 256) * min(S, 256) * 25:
        plain = (8, 2, 32, 1)
    else:
        plain = (8, 1, 64, 1)
    return plain, (8, 1, 64, 1)


def _layout_bytes(B, S, Hl, d, n, shape):
    nw, rb, kb, ks = shape
    tiles = B * Hl * -(-S // (32 * rb * nw // ks))
    nx = rb * (d // 32) * 16 + 2 * rb
    return 4096, tiles * n * (nw // ks) * nx * 64 * 4, tiles


@pytest.mark.parametrize("B,S,H,d,P", SHAPES)
def test_split_covers_every_key_tile_once_and_stays_in_the_workspace(B, S, H, d, P):
    Hl = H // P
    n = ua.key_split(B, S, H, d, P)
    assert n > 1
    total = ua.workspace_bytes(B, S, H, d, P)
    cnt_bytes = ua.workspace_count_bytes(B, S, H, d, P)
    plain, alt = _plan_shape(B, S, Hl, d, n)
    # the library's sizes identify which candidate shape the plan used
    shape = None
    for cand in (plain, alt):
        c, p, _ = _layout_bytes(B, S, Hl, d, n, cand)
        if cand[0] == 8 and c == cnt_bytes and c + p == total:
            shape = cand
            break
    assert shape is not None, "workspace size matches neither candidate shape"
    nw, rb, kb, ks = shape
    c_bytes, p_bytes, tiles = _layout_bytes(B, S, Hl, d, n, shape)
    nt_all = -(-S // kb)
    U = nt_all // ks
    assert U * ks == nt_all                      # key groups only for an even tile count
    nwg = nw // ks
    nx = rb * (d // 32) * 16 + 2 * rb
    covered = np.zeros(nt_all, np.int64)
    max_part = -1
    for split in range(n):
        u0, u1 = split * U // n, (split + 1) * U // n
        ntiles = u1 - u0
        assert ntiles >= 8
        for grp in range(ks):
            kvbase_tile = u0 * ks + grp * ntiles
            covered[kvbase_tile:kvbase_tile + ntiles] += 1
            assert kvbase_tile * kb < S                # a full first tile exists
        # partial floats this split's storing waves write for the last tile
        last = ((tiles - 1) * n + split) * nwg * nx * 64 + (nwg - 1) * nx * 64 + (nx - 1) * 64 + 63
        max_part = max(max_part, last)
    assert np.all(covered == 1)                  # every key tile exactly once per query tile
    assert tiles < 1024 and cnt_bytes >= tiles * 4  # one count per query tile
    assert cnt_bytes + (max_part + 1) * 4 == total


# ---- stream-K: the workgroups' runs, restated from the kernel and launch ----

def _sk_shapes():
    """Shapes whose *_ws calls run stream-K: the DiT-long workload, the GPU
    tests' cases, and a scan of lengths, head counts, batches and head dims."""
    out = {(1, 16384, 24, 128, 8), (1, 16384, 40, 128, 8), (2, 3000, 48, 64, 8), (1, 5000, 64, 64, 8),
           (1, 12344, 24, 128, 8)}
    for d in (64, 128):
        for S in (2000, 3000, 4104, 5000, 6000, 8000, 9999, 12000, 16000, 20000):
            for Hl in (1, 2, 3, 5, 6, 8):
                for B in (1, 2):
                    if ua.stream_k_iters(B, S, Hl * 8, d, 8):
                        out.add((B, S, Hl * 8, d, 8))
    return sorted(out)


SK_SHAPES = _sk_shapes()


def sk_items(qtiles, T, L, launched, guard=True):
    """The work items of every launched workgroup, as the kernel forms them:
    (workgroup, query tile, first key tile, key tiles, part, parts)."""
    total = qtiles * T
    items = []
    for w in range(launched):
        it, end = w * L, min((w + 1) * L, total)
        if guard and it >= end:
            continue
        while True:
            tile = it // T
            k0 = it - tile * T
            n = min(T - k0, end - it)
            first, last = tile * T // L, ((tile + 1) * T - 1) // L
            items.append((w, tile, k0, n, w - first, last - first + 1))
            it += n
            if not it < end:
                break
    return items


@pytest.mark.parametrize("B,S,H,d,P", SK_SHAPES)
def test_stream_k_runs_cover_every_iteration_once(B, S, H, d, P):
    Hl = H // P
    L = ua.stream_k_iters(B, S, H, d, P)
    n = ua.key_split(B, S, H, d, P)
    assert L >= 16 and n >= 2
    rows, kb = 256, 64                      # stream-K runs the 8-wave 256-row shape on 64-key tiles
    qtiles, T = B * Hl * -(-S // rows), -(-S // kb)
    assert qtiles < 1024                    # arrival counts fit the fixed count region
    nx = (d // 32) * 16 + 2
    assert ua.workspace_bytes(B, S, H, d, P) == 4096 + qtiles * n * 8 * nx * 64 * 4
    launched = -(-(qtiles * T) // L)        # the launch: ceil(total / L) workgroups
    assert launched <= 256
    items = sk_items(qtiles, T, L, launched)
    covered = np.zeros((qtiles, T), np.int64)
    parts = {}
    for w, tile, k0, m, part, nparts in items:
        assert 0 <= tile < qtiles and 0 <= k0 < T and 1 <= m <= T - k0
        assert 0 <= part < nparts <= n      # partial slots (tile * n + part) inside the workspace
        covered[tile, k0:k0 + m] += 1
        parts.setdefault(tile, []).append((part, nparts, k0))
    assert np.all(covered == 1)
    for tile, ps in parts.items():
        # parts numbered 0 .. nparts-1 in key order, each exactly once
        ps.sort(key=lambda p: p[2])
        assert [p[0] for p in ps] == list(range(len(ps))) and all(p[1] == len(ps) for p in ps)
    assert max(len(ps) for ps in parts.values()) == n


def test_stream_k_without_the_launch_count_and_guard_runs_out_of_range():
    # One workgroup per CU and no guard: for B=2, S=3000, 48 heads over 8
    # ranks, d=64, 256 * 27 iterations exceed the 6768 there are, and the
    # workgroups past the end take query tile 144 of 144 with a negative tile
    # count -- the out-of-range reads this layout guards against.
    L = ua.stream_k_iters(2, 3000, 48, 64, 8)
    qtiles, T = 2 * 6 * 12, 47
    assert L == 27 and 256 * L > qtiles * T
    bad = [it for it in sk_items(qtiles, T, L, 256, guard=False) if it[1] >= qtiles or it[3] < 1]
    assert bad and bad[0][1] == qtiles and bad[0][3] < 0
