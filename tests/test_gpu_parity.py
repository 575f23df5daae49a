"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Every test compares the library's output with ``oracle`` on the same seeded
inputs: values within the stated tolerance, layout bit-exact (owned slots
written, every other slot keeps the sentinel bits), and the bit-exact
cross-checks that need no tolerance (permute vs the oracle's permutation,
fused == permute(serial), run-to-run determinism).
"""
import math

import numpy as np
import pytest

import comm_fusion_amd as ua
import oracle
from gpu_helpers import (assert_close, bits_to_f64, check_dest_layout, empty_bf16, sentinel_buffer,
                         to_dev, to_host_bits)
from ua_inputs import SENTINEL_BITS, WORKLOADS, Workload, make_qkv, sampled_rows, workload_qkv

pytestmark = pytest.mark.gpu


def _sync():
    import torch
    torch.cuda.synchronize()


def _dev4(bits):
    return to_dev(bits).view(*bits.shape)


def _fused(Q, K, V, rank, P, H, scale=None):
    B, S, Hl, d = Q.shape
    dest = sentinel_buffer(B * S * H * d)
    ua.attn_ulysses_fused(_dev4(Q), _dev4(K), _dev4(V), rank, P, dest, scale)
    _sync()
    return to_host_bits(dest)


def _serial(Q, K, V, rank, P, scale=None):
    B, S, Hl, d = Q.shape
    o = empty_bf16(Q.size).view(B, S, Hl, d)
    ua.attn_serial(_dev4(Q), _dev4(K), _dev4(V), rank, P, o, scale)
    _sync()
    return o


def _compare_rows(dest_bits, Q, K, V, rows, H, P, rank, scale, what):
    B, S, Hl, d = Q.shape
    ref = oracle.attn_rows(Q, K, V, scale, rows)
    offs = oracle.dest_offsets(rows, B, S, H, d, P, rank)
    assert np.all(offs >= 0)
    got = bits_to_f64(dest_bits[offs[:, None] + np.arange(d)[None, :]])
    return assert_close(got, ref, what)


def _case(B, S, H, P, rank, d, seed):
    Q, K, V = make_qkv(B, S, H // P, d, seed)
    return Q, K, V


# Small shapes spanning several Q/KV tiles, ragged tails (S not a multiple of
# the 128-row Q tile or 64-key KV tile), regions that straddle Q tiles, both
# head dims, P = 1 (identity placement) and S = P (one row per region).
SMALL = [
    # B, S, H, P, rank, d, seed
    (1, 512, 4, 2, 0, 64, 0),      # the tiny workload
    (1, 512, 4, 2, 1, 128, 1),
    (2, 200, 8, 8, 3, 128, 2),     # ragged, regions of 25 rows
    (1, 1, 1, 1, 0, 64, 3),        # single key
    (1, 2, 2, 2, 1, 128, 4),       # S = P
    (1, 3, 2, 1, 0, 64, 5),
    (3, 130, 6, 2, 1, 64, 6),      # 130 = 2 Q tiles, 3 KV tiles (ragged)
    (1, 384, 3, 3, 2, 128, 7),     # regions of 128 rows, 3 full Q tiles
    (2, 96, 4, 4, 3, 128, 8),      # smaller than one Q tile
    # enough work units for the 8-wave, 256-row workgroups, with ragged tails
    (1, 520, 64, 1, 0, 128, 9),    # 520 = 2 full 256-row tiles + 8 rows; 8 KV tiles + 8 keys
    (2, 1030, 32, 2, 1, 64, 10),   # d = 64, regions of 515 rows
    # d = 64 with enough units of 512 rows for two row blocks per wave on
    # 32-key tiles: 1100 = 34 tiles + 12 keys, 2 units of 512 rows + 76
    (2, 1100, 64, 2, 1, 64, 13),
    # few units: two key groups of 4 waves on 32-key tiles; 1000 = 32 tiles
    # (16 per group), the last one 8 keys; units of 128 rows with a ragged last
    (2, 1000, 4, 2, 1, 128, 16),
]


@pytest.mark.parametrize("B,S,H,P,rank,d,seed", SMALL)
def test_fused_matches_oracle_and_layout(B, S, H, P, rank, d, seed):
    Q, K, V = _case(B, S, H, P, rank, d, seed)
    scale = 1.0 / math.sqrt(d)
    dest = _fused(Q, K, V, rank, P, H)
    check_dest_layout(dest, B, S, H, d, P, rank)
    rows = sampled_rows(Workload("t", B, S, H, P, rank, d, seed))
    _compare_rows(dest, Q, K, V, rows, H, P, rank, scale, "fused %s" % ((B, S, H, P, rank, d),))


@pytest.mark.parametrize("B,S,H,P,rank,d,seed", SMALL)
def test_serial_matches_oracle(B, S, H, P, rank, d, seed):
    Q, K, V = _case(B, S, H, P, rank, d, seed)
    o = to_host_bits(_serial(Q, K, V, rank, P))
    ref = oracle.attn_all(Q, K, V, 1.0 / math.sqrt(d))
    assert_close(bits_to_f64(o).reshape(ref.shape), ref, "serial")


@pytest.mark.parametrize("B,S,H,P,rank,d,seed", SMALL)
def test_permute_is_bit_exact_and_fused_equals_serial(B, S, H, P, rank, d, seed):
    Q, K, V = _case(B, S, H, P, rank, d, seed)
    o = _serial(Q, K, V, rank, P)
    dest = sentinel_buffer(B * S * H * d)
    ua.a2a_permute(o, rank, P, dest)
    _sync()
    got = to_host_bits(dest)
    want = np.full(B * S * H * d, SENTINEL_BITS, np.uint16)
    oracle.permute(to_host_bits(o).reshape(Q.shape), H, P, rank, want)
    np.testing.assert_array_equal(got, want)
    fused = _fused(Q, K, V, rank, P, H)
    np.testing.assert_array_equal(fused, got)


def test_permute_of_arbitrary_bits_is_exact():
    # Not attention output: any 16-bit patterns, including NaN/Inf codes.
    B, S, H, P, rank, d = 2, 96, 12, 4, 2, 64
    rng = np.random.default_rng(50)
    o = rng.integers(0, 1 << 16, size=(B, S, H // P, d), dtype=np.uint16)
    dest = sentinel_buffer(B * S * H * d)
    ua.a2a_permute(_dev4(o), rank, P, dest)
    _sync()
    want = np.full(B * S * H * d, SENTINEL_BITS, np.uint16)
    oracle.permute(o, H, P, rank, want)
    np.testing.assert_array_equal(to_host_bits(dest), want)


def test_all_ranks_compose_to_full_multihead_attention():
    # One global [B][S][H][d] problem; every rank runs on its head slice into
    # the same destination.  Afterwards no sentinel remains and every row
    # matches the oracle for its global head.
    B, S, H, P, d = 2, 160, 8, 4, 64
    Hl = H // P
    Qg, Kg, Vg = make_qkv(B, S, H, d, 60)
    dest = sentinel_buffer(B * S * H * d)
    for r in range(P):
        sl = np.s_[:, :, r * Hl:(r + 1) * Hl]
        q, k, v = (np.ascontiguousarray(t[sl]) for t in (Qg, Kg, Vg))
        ua.attn_ulysses_fused(_dev4(q), _dev4(k), _dev4(v), r, P, dest)
    _sync()
    got = to_host_bits(dest)
    assert not np.any(got == SENTINEL_BITS)
    ref = oracle.attn_all(Qg, Kg, Vg, 1.0 / math.sqrt(d))  # [B][S][H][d]
    assert_close(bits_to_f64(got).reshape(ref.shape), ref, "all ranks")


def test_runs_are_bitwise_deterministic():
    Q, K, V = _case(2, 700, 8, 4, 1, 128, 70)
    a = _fused(Q, K, V, 1, 4, 8)
    b = _fused(Q, K, V, 1, 4, 8)
    np.testing.assert_array_equal(a, b)


def test_uniform_v_and_zero_q_closed_forms():
    B, S, H, P, rank, d = 1, 300, 4, 2, 1, 128
    Q, K, _ = _case(B, S, H, P, rank, d, 80)
    rng = np.random.default_rng(81)
    from ua_inputs import to_bf16_bits
    c = to_bf16_bits(rng.standard_normal((B, 1, H // P, d)).astype(np.float32))
    V = np.ascontiguousarray(np.broadcast_to(c, Q.shape))
    dest = _fused(Q, K, V, rank, P, H)
    own = check_dest_layout(dest, B, S, H, d, P, rank)
    assert_close(bits_to_f64(own), np.broadcast_to(bits_to_f64(c), own.shape), "uniform V")
    # Q = 0: uniform weights, output = column mean of V.
    _, K2, V2 = _case(B, S, H, P, rank, d, 82)
    Z = np.zeros_like(K2)
    dest = _fused(Z, K2, V2, rank, P, H)
    own = check_dest_layout(dest, B, S, H, d, P, rank)
    mean = bits_to_f64(V2).mean(axis=1, keepdims=True)
    assert_close(bits_to_f64(own), np.broadcast_to(mean, own.shape), "Q = 0")


def test_scale_is_applied():
    Q, K, V = _case(1, 256, 2, 2, 0, 64, 90)
    for scale in (0.02, 0.6):
        dest = _fused(Q, K, V, 0, 2, 2, scale)
        rows = sampled_rows(Workload("t", 1, 256, 2, 2, 0, 64, 90))
        _compare_rows(dest, Q, K, V, rows, 2, 2, 0, scale, "scale %g" % scale)


def test_wide_rows_many_heads():
    # 512 local heads of d = 128: a sequence row spans 128 KiB, so the tile-copy
    # offsets reach 63 rows x 128 KiB; ragged S on the 8-wave path.
    B, S, H, P, rank, d = 1, 70, 1024, 2, 1, 128
    Q, K, V = _case(B, S, H, P, rank, d, 11)
    scale = 1.0 / math.sqrt(d)
    dest = _fused(Q, K, V, rank, P, H)
    check_dest_layout(dest, B, S, H, d, P, rank)
    rows = sampled_rows(Workload("t", B, S, H, P, rank, d, 11, sampled=True), n_per_head=8)
    _compare_rows(dest, Q, K, V, rows, H, P, rank, scale, "wide rows")


@pytest.mark.parametrize("B,S,H,P,rank,d", [
    (1, 1, 128, 1, 0, 64),     # one key and one query per head, 128 heads: two-row-block d = 64 launch
    (1, 2, 256, 2, 0, 64),     # S = P
    (1, 33, 272, 1, 0, 64),    # one full 32-key tile + 1 key, 272 heads
    (1, 1, 128, 1, 0, 128),    # one key, 128 heads: 8-wave d = 128 launch
    (1, 2, 256, 2, 1, 128),
])
def test_tiny_sequences_with_many_heads(B, S, H, P, rank, d):
    # Enough heads for the 8-wave launches even though S is tiny: almost every
    # row of a work unit lies past S, and the one K/V tile is mostly clamped.
    Q, K, V = _case(B, S, H, P, rank, d, 14)
    scale = 1.0 / math.sqrt(d)
    dest = _fused(Q, K, V, rank, P, H)
    check_dest_layout(dest, B, S, H, d, P, rank)
    rows = sampled_rows(Workload("t", B, S, H, P, rank, d, 14))
    _compare_rows(dest, Q, K, V, rows, H, P, rank, scale, "tiny S %r" % ((B, S, H, P, rank, d),))
    Xq, Xk, Xv = make_qkv(B, S, H, d, 15)
    io = sentinel_buffer(B * S * H * d)
    ua.attn_ulysses_fused_io(_dev4(Xq), _dev4(Xk), _dev4(Xv), rank, P, io)
    _sync()
    G = [oracle.gather(x, H, P, rank) for x in (Xq, Xk, Xv)]
    np.testing.assert_array_equal(to_host_bits(io), _fused(*G, rank, P, H))


# P = 2.  S = 1030 (33 tiles of 32 keys): 8-wave launch (64 heads) and 4-wave
# launch (4 heads); S = 1024 (32 tiles): two key groups, whose partial results
# with very different maxima are merged at the end.
@pytest.mark.parametrize("H,d,S", [(64, 128, 1030), (4, 64, 1030), (4, 128, 1024), (4, 64, 1024)])
@pytest.mark.parametrize("pattern", ["rising", "spikes", "offset", "tiny"])
def test_running_max_rises_and_jumps(H, d, S, pattern):
    # Scores whose running max keeps rising along the keys (K rows scaled by
    # 0.25 .. 3.25), or jumps far past it in the middle of the sequence (three
    # keys scaled by 60: against the earlier max, exp of such a score
    # overflows fp32 for a few percent of the rows).  The online softmax has to
    # raise its max and rescale in the middle KV tiles, not only at the ends.
    # Also: every key shifted by a common vector (scores of a row sit up to a
    # few hundred away from zero, far outside exp's fp32 range), and keys
    # scaled down to ~1e-3 (nearly uniform weights).
    from ua_inputs import to_bf16_bits
    B, P, rank = 1, 2, 1
    Q, K, V = _case(B, S, H, P, rank, d, 12)
    Kf = bits_to_f64(K)
    if pattern == "rising":
        Kf *= (0.25 + 3.0 * np.arange(S) / S)[None, :, None, None]
    elif pattern == "spikes":
        for j in (200, 611, 777):
            Kf[:, j] *= 60.0
    elif pattern == "offset":
        Kf += 24.0 * np.sign(bits_to_f64(Q).mean(axis=1, keepdims=True))
    else:
        Kf *= 1e-3
    K = to_bf16_bits(Kf.astype(np.float32))
    scale = 1.0 / math.sqrt(d)
    dest = _fused(Q, K, V, rank, P, H)
    check_dest_layout(dest, B, S, H, d, P, rank)
    rows = sampled_rows(Workload("t", B, S, H, P, rank, d, 12, sampled=True), n_per_head=96)
    _compare_rows(dest, Q, K, V, rows, H, P, rank, scale, pattern)


@pytest.mark.parametrize("B,S,H,P,rank,d", [
    (1, 524290, 2, 2, 1, 64),    # 2^19 + 2 keys: 16385 tiles of 32 keys, the last holding 2
    (1, 262150, 2, 2, 0, 128),   # 2^18 + 6 keys: 4097 tiles of 64 keys, the last holding 6
])
def test_very_long_sequences(B, S, H, P, rank, d):
    # Sequences well past the benchmarked ones, with one local head: tile and
    # row indices far beyond the workloads', ragged last Q and KV tiles.
    # Sampled rows against the oracle, the full-buffer layout, and the
    # fused-io call bit-equal to gather + fused.
    seed = 16
    Q, K, V = _case(B, S, H, P, rank, d, seed)
    dest = _fused(Q, K, V, rank, P, H)
    check_dest_layout(dest, B, S, H, d, P, rank)
    rows = sampled_rows(Workload("t", B, S, H, P, rank, d, seed, sampled=True), n_per_head=16)
    _compare_rows(dest, Q, K, V, rows, H, P, rank, 1.0 / math.sqrt(d), "S = %d" % S)
    Xq, Xk, Xv = make_qkv(B, S, H, d, seed + 1)
    io = sentinel_buffer(B * S * H * d)
    ua.attn_ulysses_fused_io(_dev4(Xq), _dev4(Xk), _dev4(Xv), rank, P, io)
    _sync()
    G = [oracle.gather(x, H, P, rank) for x in (Xq, Xk, Xv)]
    np.testing.assert_array_equal(to_host_bits(io), _fused(*G, rank, P, H))


@pytest.mark.parametrize("name", ["dit_image", "dit_long", "video_dit", "mixed"])
def test_workloads_at_full_size(name):
    # The configurations the benchmark times, at full size: sampled rows
    # against the oracle (all rows for DiT image) and a full-buffer layout scan.
    w = WORKLOADS[name]
    Q, K, V = workload_qkv(w)
    dest = _fused(Q, K, V, w.rank, w.P, w.H)
    check_dest_layout(dest, w.B, w.S, w.H, w.d, w.P, w.rank)
    rows = sampled_rows(w)
    _compare_rows(dest, Q, K, V, rows, w.H, w.P, w.rank, 1.0 / math.sqrt(w.d), name)


# ---- both exchanges fused: the attention kernel reads this rank's heads in
# place from the sequence-partitioned inputs of the pre-attention exchange
# ([B][P][S/P][H][d], the same bytes as [B][S][H][d]).

IO_CASES = [
    # B, S, H, P, rank, d, seed
    (1, 512, 4, 2, 1, 64, 20),
    (2, 200, 8, 8, 3, 128, 21),      # ragged, regions of 25 rows
    (1, 520, 64, 1, 0, 128, 22),     # P = 1; 8-wave launch with ragged tails
    (1, 1032, 96, 3, 2, 128, 23),    # 8-wave launch (Hl = 32), regions of 344 rows
    (2, 1030, 32, 2, 1, 64, 24),     # d = 64, 8-wave launch
]


@pytest.mark.parametrize("B,S,H,P,rank,d,seed", IO_CASES)
def test_gather_is_bit_exact(B, S, H, P, rank, d, seed):
    X, _, _ = make_qkv(B, S, H, d, seed)
    want = oracle.gather(X, H, P, rank)
    got = empty_bf16(want.size).view(B, S, H // P, d)
    ua.a2a_gather(_dev4(X), rank, P, got)
    _sync()
    np.testing.assert_array_equal(to_host_bits(got).reshape(want.shape), want)


@pytest.mark.parametrize("B,S,H,P,rank,d,seed", IO_CASES)
def test_fused_io_matches_oracle_and_gather_then_fused(B, S, H, P, rank, d, seed):
    Xq, Xk, Xv = make_qkv(B, S, H, d, seed)
    Q, K, V = (oracle.gather(x, H, P, rank) for x in (Xq, Xk, Xv))
    dest = sentinel_buffer(B * S * H * d)
    ua.attn_ulysses_fused_io(_dev4(Xq), _dev4(Xk), _dev4(Xv), rank, P, dest)
    _sync()
    got = to_host_bits(dest)
    check_dest_layout(got, B, S, H, d, P, rank)
    rows = sampled_rows(Workload("t", B, S, H, P, rank, d, seed, sampled=True), n_per_head=64)
    _compare_rows(got, Q, K, V, rows, H, P, rank, 1.0 / math.sqrt(d), "fused io")
    # the same bits as the fused call on the gathered inputs
    np.testing.assert_array_equal(got, _fused(Q, K, V, rank, P, H))


@pytest.mark.parametrize("name", ["dit_long", "video_dit", "mixed"])
def test_fused_io_at_full_size_reads_only_this_ranks_heads(name):
    # The rank's Q, K, V placed into sequence-partitioned buffers whose other
    # heads hold NaN bits: the output must be bit-identical to the fused call
    # on the local tensors (itself checked against the oracle above), so no
    # other head is ever read.
    import torch
    w = WORKLOADS[name]
    Q, K, V = workload_qkv(w)
    lo, hi = w.rank * w.Hl, (w.rank + 1) * w.Hl
    xs = []
    for t in (Q, K, V):
        X = torch.full((w.B, w.S, w.H, w.d), float("nan"), dtype=torch.bfloat16, device="cuda")
        X[:, :, lo:hi] = _dev4(t)
        xs.append(X)
    a = sentinel_buffer(w.B * w.S * w.H * w.d)
    b = sentinel_buffer(w.B * w.S * w.H * w.d)
    ua.attn_ulysses_fused_io(xs[0], xs[1], xs[2], w.rank, w.P, a)
    ua.attn_ulysses_fused(_dev4(Q), _dev4(K), _dev4(V), w.rank, w.P, b)
    _sync()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    del xs
