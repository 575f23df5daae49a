"""GPU parity of the calls with a workspace (attn_ulysses_fused_ws,
attn_serial_ws), whose launches split each query tile's keys over several
workgroups when the query tiles are fewer than the CUs.

Every case asserts that the split really happens, then checks the output
against the fp64 oracle (values within the stated tolerance, layout
bit-exact), that attn_serial_ws + a2a_permute writes exactly the fused bytes,
that a second call on the same workspace returns the same bits, and that the
arrival counts are back at zero afterwards.
"""
import math

import numpy as np
import pytest

import comm_fusion_amd as ua
import oracle
from gpu_helpers import (assert_close, bits_to_f64, check_dest_layout, empty_bf16, sentinel_buffer,
                         to_dev, to_host_bits)
from ua_inputs import WORKLOADS, Workload, make_qkv, sampled_rows, to_bf16_bits, workload_qkv

pytestmark = pytest.mark.gpu


def _sync():
    import torch
    torch.cuda.synchronize()


def _dev4(bits):
    return to_dev(bits).view(*bits.shape)


def _fused_ws(q, k, v, rank, P, H, ws):
    B, S, Hl, d = q.shape
    dest = sentinel_buffer(B * S * H * d)
    ua.attn_ulysses_fused_ws(q, k, v, rank, P, dest, ws)
    _sync()
    return to_host_bits(dest)


def _check_split_call(Q, K, V, H, P, rank, rows, what):
    B, S, Hl, d = Q.shape
    q, k, v = _dev4(Q), _dev4(K), _dev4(V)
    ws = ua.new_workspace(B, S, H, d, P, q.device)
    assert ws is not None and ws.numel() == ua.workspace_bytes(B, S, H, d, P)
    dest = _fused_ws(q, k, v, rank, P, H, ws)
    check_dest_layout(dest, B, S, H, d, P, rank)
    ref = oracle.attn_rows(Q, K, V, 1.0 / math.sqrt(d), rows)
    offs = oracle.dest_offsets(rows, B, S, H, d, P, rank)
    err = assert_close(bits_to_f64(dest[offs[:, None] + np.arange(d)[None, :]]), ref, what)
    # the serial form with the same split writes exactly the fused bytes
    o = empty_bf16(Q.size).view(B, S, Hl, d)
    ua.attn_serial_ws(q, k, v, rank, P, o, ws)
    dest2 = sentinel_buffer(B * S * H * d)
    ua.a2a_permute(o, rank, P, dest2)
    _sync()
    np.testing.assert_array_equal(to_host_bits(dest2), dest)
    # the counts were reset: a second call on the same workspace, same bits
    np.testing.assert_array_equal(_fused_ws(q, k, v, rank, P, H, ws), dest)
    cnt = ws[:ua.workspace_count_bytes(B, S, H, d, P)].cpu().numpy()
    assert not cnt.any(), "arrival counts not reset"
    return err


# B, S, H, P, rank, d, seed, expected key split
SPLIT_CASES = [
    (1, 4096, 24, 8, 3, 128, 41, 2),   # the DiT-image shape: two key groups of 4 waves, 96 tiles
    (1, 8176, 8, 8, 2, 128, 42, 4),    # ragged: last query tile 112 rows, last key tile 16 keys; key groups
    (2, 2048, 8, 2, 1, 64, 43, 2),     # d = 64 with key groups, B = 2
    (1, 8192, 40, 8, 0, 64, 44, 3),    # d = 64, one row block per wave, parts of 42, 43, 43 tiles
    (1, 16384, 48, 8, 1, 64, 45, 4),   # d = 64, two row blocks per wave
    (1, 3584, 8, 8, 1, 64, 51, 4),     # d = 64 with key groups, parts of 14 tile pairs
    (1, 4064, 8, 8, 6, 128, 52, 4),    # plain call on one wave per SIMD; split on the 8-wave shape, ragged last key tile
    (1, 16384, 40, 8, 7, 128, 54, 2),  # 320 tiles (1.25 rounds unsplit): stream-K, 320 iterations per workgroup
    (1, 32768, 40, 8, 2, 128, 55, 2),  # 640 tiles (2.5 rounds unsplit): five full rounds
]


@pytest.mark.parametrize("B,S,H,P,rank,d,seed,n", SPLIT_CASES)
def test_key_split_matches_oracle_and_serial(B, S, H, P, rank, d, seed, n):
    print("key split case", (B, S, H, P, rank, d, seed), flush=True)
    assert ua.key_split(B, S, H, d, P) == n
    Q, K, V = make_qkv(B, S, H // P, d, seed)
    w = Workload("t", B, S, H, P, rank, d, seed, sampled=S > 4096)
    _check_split_call(Q, K, V, H, P, rank, sampled_rows(w, n_per_head=64), "split %s" % ((B, S, H, d),))


def test_key_split_merges_parts_with_far_apart_maxima():
    # Key norms grow along the sequence (x0.25 at key 0 to x4 at the end), so
    # the last part's running max exceeds the first's by ~20 in the log2
    # domain: the merge must rescale the early parts by ~2^-20, not drop or
    # overflow them.
    B, S, H, P, rank, d = 1, 8192, 8, 8, 5, 128
    assert ua.key_split(B, S, H, d, P) == 4
    Q, K, V = make_qkv(B, S, H // P, d, 46)
    f = (0.25 + 3.75 * np.arange(S) / (S - 1)).astype(np.float32)[None, :, None, None]
    Kf = (K.astype(np.uint32) << 16).view(np.float32) * f
    K = to_bf16_bits(Kf)
    w = Workload("t", B, S, H, P, rank, d, 46, sampled=True)
    _check_split_call(Q, K, V, H, P, rank, sampled_rows(w, n_per_head=128), "far-apart maxima")


@pytest.mark.parametrize("name", ["dit_image", "dit_long"])
def test_workloads_with_key_split_at_full_size(name):
    # The two configurations with fewer query tiles than CUs, at full size:
    # all rows of DiT image, sampled rows of DiT long (peaky keys).
    w = WORKLOADS[name]
    print("key split workload", name, flush=True)
    assert ua.key_split(w.B, w.S, w.H, w.d, w.P) > 1
    Q, K, V = workload_qkv(w)
    _check_split_call(Q, K, V, w.H, w.P, w.rank, sampled_rows(w), name)


def test_workspace_call_without_split_is_the_plain_call():
    # Shapes the plain launch already serves best (too short; 256 query tiles,
    # one full round over the CUs): no split, the workspace is not needed and
    # the output is the plain call's, bit for bit.
    for (B, S, H, P, rank, d) in [(1, 512, 4, 2, 0, 64), (1, 4096, 128, 8, 7, 128)]:
        assert ua.key_split(B, S, H, d, P) == 1 and ua.workspace_bytes(B, S, H, d, P) == 0
        Q, K, V = make_qkv(B, S, H // P, d, 47)
        q, k, v = _dev4(Q), _dev4(K), _dev4(V)
        a = _fused_ws(q, k, v, rank, P, H, None)
        dest = sentinel_buffer(B * S * H * d)
        ua.attn_ulysses_fused(q, k, v, rank, P, dest)
        _sync()
        np.testing.assert_array_equal(a, to_host_bits(dest))


def test_split_and_unsplit_calls_agree_to_rounding():
    # Same inputs, with and without the workspace: both near the oracle, and
    # elementwise within a few bf16 steps of each other.
    B, S, H, P, rank, d = 1, 8192, 8, 8, 2, 128
    Q, K, V = make_qkv(B, S, H // P, d, 48)
    q, k, v = _dev4(Q), _dev4(K), _dev4(V)
    ws = ua.new_workspace(B, S, H, d, P, q.device)
    a = bits_to_f64(_fused_ws(q, k, v, rank, P, H, ws))
    dest = sentinel_buffer(B * S * H * d)
    ua.attn_ulysses_fused(q, k, v, rank, P, dest)
    _sync()
    b = bits_to_f64(to_host_bits(dest))
    Hl = H // P
    a4 = a.reshape(B, S, H, d)[:, :, rank * Hl:(rank + 1) * Hl]
    b4 = b.reshape(B, S, H, d)[:, :, rank * Hl:(rank + 1) * Hl]
    diff = np.abs(a4 - b4)
    assert diff.max() <= 4 * 2.0 ** -8 * max(np.abs(b4).max(), 1e-3), diff.max()


def test_fused_io_with_key_split_equals_gather_then_fused():
    # Both exchanges fused, split launch: reading this rank's heads in place
    # from [B][P][S/P][H][d] gives the bytes of a2a_gather + attn_ulysses_fused_ws.
    B, S, H, P, rank, d = 1, 4096, 24, 8, 6, 128
    assert ua.key_split(B, S, H, d, P) == 2
    Xq, Xk, Xv = (_dev4(x) for x in make_qkv(B, S, H, d, 50))
    ws = ua.new_workspace(B, S, H, d, P, Xq.device)
    io = sentinel_buffer(B * S * H * d)
    ua.attn_ulysses_fused_io_ws(Xq, Xk, Xv, rank, P, io, ws)
    loc = [empty_bf16(B * S * (H // P) * d).view(B, S, H // P, d) for _ in range(3)]
    for X, L in zip((Xq, Xk, Xv), loc):
        ua.a2a_gather(X, rank, P, L)
    ref = _fused_ws(*loc, rank, P, H, ws)
    np.testing.assert_array_equal(to_host_bits(io), ref)
    check_dest_layout(ref, B, S, H, d, P, rank)


def test_all_ranks_with_key_split_compose_to_full_multihead_attention():
    # One global [B][S][H][d] problem; every rank runs its split call on its
    # head slice into one destination, each rank with its own workspace.
    # Afterwards no sentinel remains and sampled rows of every global head
    # match the oracle.
    import torch
    B, S, H, P, d = 1, 4096, 16, 8, 128
    Hl = H // P
    assert ua.key_split(B, S, H, d, P) > 1
    Qg, Kg, Vg = make_qkv(B, S, H, d, 53)
    dest = sentinel_buffer(B * S * H * d)
    for r in range(P):
        sl = np.s_[:, :, r * Hl:(r + 1) * Hl]
        q, k, v = (_dev4(np.ascontiguousarray(t[sl])) for t in (Qg, Kg, Vg))
        ws = ua.new_workspace(B, S, H, d, P, q.device)
        ua.attn_ulysses_fused_ws(q, k, v, r, P, dest, ws)
    torch.cuda.synchronize()
    got = to_host_bits(dest)
    assert not np.any(got == np.uint16(0x7FD5))
    w = Workload("t", B, S, H, 1, 0, d, 53, sampled=True)
    rows = sampled_rows(w, n_per_head=32)
    ref = oracle.attn_rows(Qg, Kg, Vg, 1.0 / math.sqrt(d), rows)     # rows of all H heads
    offs = oracle.dest_offsets(rows, B, S, H, d, 1, 0)                # P = 1: plain [B][S][H][d]
    assert_close(bits_to_f64(got[offs[:, None] + np.arange(d)[None, :]]), ref, "all ranks, split")


def test_one_workspace_serves_shapes_in_turn():
    # A workspace sized for the larger shape serves a smaller one in between:
    # every call leaves the arrival counts at zero, and the results equal the
    # same calls on fresh workspaces, bit for bit.
    big = WORKLOADS["dit_long"]
    small = WORKLOADS["dit_image"]
    assert ua.workspace_bytes(big.B, big.S, big.H, big.d, big.P) >= \
        ua.workspace_bytes(small.B, small.S, small.H, small.d, small.P) > 0
    ins = {}
    for w in (big, small):
        ins[w.name] = [_dev4(x) for x in workload_qkv(w)]
    shared = ua.new_workspace(big.B, big.S, big.H, big.d, big.P, ins[big.name][0].device)
    got = []
    for w in (big, small, big):
        got.append(_fused_ws(*ins[w.name], w.rank, w.P, w.H, shared))
    for w, g in zip((big, small, big), got):
        fresh = ua.new_workspace(w.B, w.S, w.H, w.d, w.P, ins[w.name][0].device)
        np.testing.assert_array_equal(g, _fused_ws(*ins[w.name], w.rank, w.P, w.H, fresh))
