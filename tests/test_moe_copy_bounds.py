"""Host-side bounds check of the MoE tile kernel's global reads and writes (no GPU).

The kernel addresses its operand copies as a wave-uniform base plus a 32-bit
per-lane byte offset: weight rows of the tile's expert (Linear-1's gate and up
rows arranged so each wave holds matching columns), token rows gathered
through row_slot (Linear-1 reads x at slot / k, Linear-2 reads act at the
receive row; rows past an expert's end repeat its last row).  This test
restates that addressing (which 1 KiB copies each wave issues, which row and
16-byte chunk each lane fetches, the k offset of every step) and the two
epilogues' stores (Linear-1 into act, Linear-2 into the Combine slots or the
receive rows), and checks for every tile of the five MoE workloads, of the
ragged-expert case of the GPU tests and of shapes at the size limits that
every 16-byte access lies inside its buffer and that no 32-bit offset wraps.
A mutant that takes Linear-2's k length from hidden instead of inter is
shown to read out of bounds.  For an expert's partial last tile, the waves
that skip their token copies and their padded token blocks are checked to
leave every row that is read copied and every valid row computed.
"""
import numpy as np
import pytest

import comm_fusion_amd as ua
from moe_inputs import MOE_WORKLOADS, MoeWorkload, moe_tokens

BM, BF, BK, NW = 256, 256, 64, 8
NCPW = BF * BK * 2 // 1024 // NW   # 1 KiB copies per wave per operand tile
L1_COLS, L2_COLS = 128, 256
U32 = 1 << 32


def lanes():
    wave = np.arange(NW)[:, None, None]
    i = np.arange(NCPW)[None, :, None]
    lane = np.arange(64)[None, None, :]
    c = NCPW * wave + i
    r = 8 * c + (lane >> 3)                                   # tile row of the lane's chunk
    chunk16 = ((lane & 7) ^ (4 * (i & 1) + (lane >> 4))) * 16  # byte offset of the fetched chunk
    return np.broadcast_arrays(r, chunk16)


def tile_accesses(kind, rows, row0, row_slot, m, n, hidden, inter, k, k_len=None):
    """(weight read offsets, token read rows/offsets, max k offset) of one tile."""
    K = (hidden if kind == 0 else inter) if k_len is None else k_len
    r, chunk16 = lanes()
    h, q = r >> 7, r & 127
    if kind == 0:
        wrow = np.where(q < 64, L1_COLS * n + 64 * h + q, inter + L1_COLS * n + 64 * h + q - 64)
    else:
        wrow = L2_COLS * n + r
    aoff = wrow.astype(np.int64) * K * 2 + chunk16
    rl = np.minimum(m * BM + r, rows - 1)
    ri = row0 + rl
    brow = (row_slot[ri] // k) if kind == 0 else ri
    boff = brow.astype(np.int64) * K * 2 + chunk16
    kmax = (K // BK - 1) * BK * 2
    return aoff, boff, kmax


def check_problem(P, T, hidden, inter, E, k, offsets, row_slot, k_len_l2=None):
    E_l = E // P
    N = int(offsets[-1])
    w1_bytes = 2 * inter * hidden * 2          # one expert's W1
    w2_bytes = hidden * inter * 2
    x_bytes = P * T * hidden * 2
    act_bytes = N * inter * 2
    comb_bytes = P * T * k * hidden * 2
    bad = []
    for e in range(E_l):
        row0, rows = int(offsets[e]), int(offsets[e + 1] - offsets[e])
        if rows == 0:
            continue
        mt = -(-rows // BM)
        for kind, nt in ((0, inter // L1_COLS), (1, hidden // L2_COLS)):
            for m in range(mt):
                for n in range(nt):
                    aoff, boff, kmax = tile_accesses(kind, rows, row0, row_slot, m, n, hidden, inter, k,
                                                     k_len_l2 if kind == 1 else None)
                    wlim = w1_bytes if kind == 0 else w2_bytes
                    blim = x_bytes if kind == 0 else act_bytes
                    for name, off, lim in (("weights", aoff, wlim), ("tokens", boff, blim)):
                        if off.min() < 0 or off.max() >= U32 or off.max() + kmax + 16 > lim:
                            bad.append((e, kind, m, n, name))
                    # epilogue stores of the tile's valid rows
                    tr = np.arange(BM)
                    valid = m * BM + tr < rows
                    ri = row0 + m * BM + tr[valid]
                    if kind == 0:
                        # act[row][128 n + 0 .. 127], 8-byte stores
                        last = ri.astype(np.int64) * inter * 2 + (L1_COLS * n + L1_COLS) * 2
                        if last.max() > act_bytes:
                            bad.append((e, kind, m, n, "act store"))
                    else:
                        slot = row_slot[ri].astype(np.int64)
                        if slot.min() < 0 or (slot.max() + 1) * hidden * 2 > comb_bytes:
                            bad.append((e, kind, m, n, "combine store"))
                        if (L2_COLS * n + L2_COLS) * 2 > hidden * 2:
                            bad.append((e, kind, m, n, "combine columns"))
    return bad


def _layout(idx, rank, P, hidden, inter, E):
    off, slots = ua.moe_recv_layout(idx, rank, P, hidden, inter, E)
    return np.asarray(off, np.int64), np.asarray(slots, np.int64)


@pytest.mark.parametrize("name", sorted(MOE_WORKLOADS))
def test_every_access_of_the_workloads_is_in_bounds(name):
    w = MOE_WORKLOADS[name]
    _, idx, _ = moe_tokens(w)
    off, slots = _layout(idx, w.rank, w.P, w.hidden, w.inter, w.E)
    assert check_problem(w.P, w.T, w.hidden, w.inter, w.E, w.k, off, slots) == []


def _routing(P, T, E, k, rank, counts, seed):
    """Routing where rank's local experts get exactly `counts` rows (first
    choices of distinct tokens); every other choice goes to other ranks'
    experts, distinct within a token (with one rank, counts cover every token
    and k is 1)."""
    rng = np.random.default_rng(seed)
    E_l = E // P
    other = np.array([g for g in range(E) if g // E_l != rank], np.int64)
    assert len(counts) == E_l and (len(other) >= k or (P == 1 and k == 1 and sum(counts) == T))
    idx = np.zeros((P * T, k), np.int64)
    for t in range(P * T):
        if len(other):
            idx[t] = rng.choice(other, size=k, replace=False)
    pool = rng.permutation(P * T)
    pos = 0
    for e, c in enumerate(counts):
        idx[pool[pos:pos + c], 0] = rank * E_l + e
        pos += c
    return idx.astype(np.int32).reshape(P, T, k)


@pytest.mark.parametrize("P,T,hidden,inter,E,k,counts", [
    (2, 400, 256, 128, 12, 2, [0, 1, 127, 128, 129, 300]),     # the ragged-expert GPU case
    (2, 600, 512, 256, 8, 2, [255, 256, 257, 0]),
    (1, 1024, 256, 128, 2, 1, [1024, 0]),                     # one expert holds every token
])
def test_ragged_experts_are_in_bounds(P, T, hidden, inter, E, k, counts):
    rank = P - 1
    idx = _routing(P, T, E, k, rank, counts, seed=sum(counts))
    off, slots = _layout(idx, rank, P, hidden, inter, E)
    assert list(np.diff(off)) == counts
    assert check_problem(P, T, hidden, inter, E, k, off, slots) == []


def test_offsets_at_the_size_limits_do_not_wrap():
    # one expert's W1 just under 2^32 bytes is rejected by the host (2 inter
    # hidden 2 < 2^32 is required); the largest accepted shape keeps every
    # weight offset below 2^32
    hidden, inter = 16384, 32768 - 128
    assert 2 * inter * hidden * 2 < U32
    r, chunk16 = lanes()
    n = inter // L1_COLS - 1
    h, q = r >> 7, r & 127
    wrow = np.where(q < 64, L1_COLS * n + 64 * h + q, inter + L1_COLS * n + 64 * h + q - 64)
    aoff = wrow.astype(np.int64) * hidden * 2 + chunk16
    assert aoff.max() + (hidden // BK - 1) * BK * 2 + 16 <= 2 * inter * hidden * 2 < U32


def test_mutant_with_the_wrong_k_length_reads_out_of_bounds():
    w = MOE_WORKLOADS["moe_small"]
    _, idx, _ = moe_tokens(w)
    off, slots = _layout(idx, w.rank, w.P, w.hidden, w.inter, w.E)
    bad = check_problem(w.P, w.T, w.hidden, w.inter, w.E, w.k, off, slots, k_len_l2=w.hidden)
    assert bad and all(b[1] == 1 for b in bad)


def partial_tile_plan(vrows):
    """Restates the kernel's partial-tile rule for a tile holding `vrows`
    valid token rows: wave (wf, wt) = (wave % 2, wave // 2) computes token
    blocks wt and wt + 4 (32 rows each) while they start below vrows; wave w
    copies token rows 32 w .. 32 w + 31 only while 32 w < vrows.  Returns
    (rows read by the fragment reads, rows copied, rows computed)."""
    read, copied, computed = set(), set(), set()
    for wave in range(NW):
        wt = wave >> 1
        nb = int(32 * wt < vrows) + int(128 + 32 * wt < vrows)
        for tb in range(nb):                        # blocks wt, then wt + 4
            rows = range(32 * (wt + 4 * tb), 32 * (wt + 4 * tb) + 32)
            read.update(rows)
            computed.update(rows)
        if 32 * wave < vrows:
            copied.update(range(32 * wave, 32 * wave + 32))
    return read, copied, computed


@pytest.mark.parametrize("vrows", list(range(1, BM + 1)))
def test_partial_tiles_read_only_copied_rows_and_compute_every_row(vrows):
    read, copied, computed = partial_tile_plan(vrows)
    assert read <= copied
    assert set(range(vrows)) <= computed
    # padded blocks are skipped: at most the 31 rows past vrows that share
    # the last valid block are computed
    assert max(computed) < vrows + 31 and len(computed) == 32 * -(-vrows // 32)


def test_partial_tile_plan_catches_a_wrong_block_map():
    # the mapping before the interleave (blocks 2 wt, 2 wt + 1) with the
    # same copy rule would leave valid rows uncomputed
    def old(vrows):
        computed = set()
        for wave in range(NW):
            wt = wave >> 1
            nb = int(32 * wt < vrows) + int(128 + 32 * wt < vrows)
            for tb in range(nb):
                computed.update(range(64 * wt + 32 * tb, 64 * wt + 32 * tb + 32))
        return computed
    assert any(not set(range(v)) <= old(v) for v in range(1, BM + 1))
