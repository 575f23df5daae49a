"""Seeded sweeps of random valid shapes through every entry point (GPU).

Shapes are drawn once from a fixed seed: batch 1-3, P in {1, 2, 3, 4, 5, 8}
(any rank), S a multiple of P that is mostly ragged against the 64-key and
128/256-row tiles, both head dims, and enough heads on some draws for the
8-wave launch.  Each shape is checked against the oracle on sampled rows, for
the exact destination layout, and for bit equality between the fused call,
the serial attention + permute, and the fused call on sequence-partitioned
inputs.  A third sweep does the same for the calls with a workspace on shapes
whose query tiles are few enough for a key split.

UA_SWEEP_WIDE=1 in the environment swaps in wider draws from other seeds
(150 + 60 shapes for the plain calls, 60 for the key split) for a longer run.
"""
import math
import os

import numpy as np
import pytest

import comm_fusion_amd as ua
import oracle
from gpu_helpers import (assert_close, bits_to_f64, check_dest_layout, empty_bf16, sentinel_buffer,
                         to_dev, to_host_bits)
from ua_inputs import Workload, make_qkv, sampled_rows

pytestmark = pytest.mark.gpu


def sweep_shapes(n=32, seed=2026):
    """(B, S, H, P, rank, d, seed) tuples.  Every third draw has enough work
    units (B*Hl*ceil(S/256) >= 128) for the 8-wave launch.  Bounded to 2.5e7
    elements per input and 1e10 multiply-adds per shape."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        wide = len(out) % 3 == 2
        d = int(rng.choice([64, 128]))
        P = int(rng.choice([1, 2, 3, 4, 5, 8]))
        Hl = int(rng.choice([33, 40, 64] if wide else [1, 2, 3, 5, 8, 33]))
        B = int(rng.integers(1, 4))
        S = P * int(rng.integers(1, 1 + 1400 // P))
        if B * S * Hl * P * d > 2.5e7 or B * Hl * S * S * d > 1e10:
            continue
        if wide and B * Hl * -(-S // 256) < 128:
            continue
        out.append((B, S, Hl * P, P, int(rng.integers(0, P)), d, 100 + len(out)))
    return out


WIDE = os.environ.get("UA_SWEEP_WIDE") == "1"
SHAPES = sweep_shapes(150, 9101) if WIDE else sweep_shapes()


def sweep_shapes_b(n=16, seed=2027):
    """Shapes aimed at the two launch shapes with extra structure: even draws
    are d = 64 with enough 512-row units for two row blocks per wave (units
    halve against 256-row ones: B*Hl*ceil(S/512) >= 128 and fewer rounds over
    256 CUs), odd draws have fewer than 128 units of 256 rows and an even
    32-key tile count (two key groups per workgroup)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        P = int(rng.choice([1, 2, 3, 4]))
        B = int(rng.integers(1, 3))
        if len(out) % 2 == 0:
            d, Hl = 64, int(rng.choice([40, 64, 96]))
            S = P * int(rng.integers(700 // P, 1 + 1400 // P))
            u512, u256 = B * Hl * -(-S // 512), B * Hl * -(-S // 256)
            if u512 < 128 or -(-u512 // 256) * 2 > -(-u256 // 256):
                continue
        else:
            d, Hl = int(rng.choice([64, 128])), int(rng.choice([1, 2, 3]))
            S = P * int(rng.integers(1, 1 + 1500 // P))
            nt = -(-S // 32)
            if B * Hl * -(-S // 256) >= 128 or nt < 2 or nt % 2:
                continue
        if B * S * Hl * P * d > 2.5e7:
            continue
        out.append((B, S, Hl * P, P, int(rng.integers(0, P)), d, 300 + len(out)))
    return out


SHAPES_B = sweep_shapes_b(60, 9102) if WIDE else sweep_shapes_b()


def sweep_shapes_split(n=12, seed=2028):
    """Shapes for the calls with a workspace (key split): few query tiles
    (B*Hl*ceil(S/128) <= 96) and 2048-12000 keys, mostly ragged against the
    tiles, both head dims, any P and rank; bounded like the other sweeps."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        d = int(rng.choice([64, 128]))
        P = int(rng.choice([1, 2, 3, 4, 8]))
        Hl = int(rng.choice([1, 2, 3]))
        B = int(rng.integers(1, 3))
        S = P * int(rng.integers(2048 // P, 1 + 12000 // P))
        if B * Hl * -(-S // 128) > 96 or B * S * Hl * P * d > 2.5e7:
            continue
        out.append((B, S, Hl * P, P, int(rng.integers(0, P)), d, 500 + len(out)))
    return out


SHAPES_SPLIT = sweep_shapes_split(60, 9103) if WIDE else sweep_shapes_split()


def _dev(a):
    return to_dev(a).view(*a.shape)


@pytest.mark.parametrize("B,S,H,P,rank,d,seed", SHAPES + SHAPES_B)
def test_sweep(B, S, H, P, rank, d, seed):
    import torch
    Hl = H // P
    Xq, Xk, Xv = make_qkv(B, S, H, d, seed)           # sequence-partitioned inputs
    Q, K, V = (oracle.gather(x, H, P, rank) for x in (Xq, Xk, Xv))
    q, k, v = _dev(Q), _dev(K), _dev(V)
    n = B * S * H * d
    fused, io, serial = sentinel_buffer(n), sentinel_buffer(n), sentinel_buffer(n)
    o_local = empty_bf16(Q.size).view(B, S, Hl, d)
    ua.attn_ulysses_fused(q, k, v, rank, P, fused)
    ua.attn_ulysses_fused_io(_dev(Xq), _dev(Xk), _dev(Xv), rank, P, io)
    ua.attn_serial(q, k, v, rank, P, o_local)
    ua.a2a_permute(o_local, rank, P, serial)
    torch.cuda.synchronize()
    got = to_host_bits(fused)
    check_dest_layout(got, B, S, H, d, P, rank)
    np.testing.assert_array_equal(got, to_host_bits(serial))
    np.testing.assert_array_equal(got, to_host_bits(io))
    rows = sampled_rows(Workload("sweep", B, S, H, P, rank, d, seed, sampled=True), n_per_head=16)
    ref = oracle.attn_rows(Q, K, V, 1.0 / math.sqrt(d), rows)
    offs = oracle.dest_offsets(rows, B, S, H, d, P, rank)
    assert np.all(offs >= 0)
    assert_close(bits_to_f64(got[offs[:, None] + np.arange(d)[None, :]]), ref, "sweep %r" % ((B, S, H, P, rank, d),))


@pytest.mark.parametrize("B,S,H,P,rank,d,seed", SHAPES_SPLIT)
def test_sweep_key_split(B, S, H, P, rank, d, seed):
    import torch
    Hl = H // P
    assert ua.key_split(B, S, H, d, P) > 1
    Xq, Xk, Xv = make_qkv(B, S, H, d, seed)
    Q, K, V = (oracle.gather(x, H, P, rank) for x in (Xq, Xk, Xv))
    q, k, v = _dev(Q), _dev(K), _dev(V)
    ws = ua.new_workspace(B, S, H, d, P, q.device)
    n = B * S * H * d
    fused, io, serial = sentinel_buffer(n), sentinel_buffer(n), sentinel_buffer(n)
    o_local = empty_bf16(Q.size).view(B, S, Hl, d)
    ua.attn_ulysses_fused_ws(q, k, v, rank, P, fused, ws)
    ua.attn_ulysses_fused_io_ws(_dev(Xq), _dev(Xk), _dev(Xv), rank, P, io, ws)
    ua.attn_serial_ws(q, k, v, rank, P, o_local, ws)
    ua.a2a_permute(o_local, rank, P, serial)
    torch.cuda.synchronize()
    got = to_host_bits(fused)
    check_dest_layout(got, B, S, H, d, P, rank)
    np.testing.assert_array_equal(got, to_host_bits(serial))
    np.testing.assert_array_equal(got, to_host_bits(io))
    assert not ws[:ua.workspace_count_bytes(B, S, H, d, P)].cpu().numpy().any()
    rows = sampled_rows(Workload("sweep", B, S, H, P, rank, d, seed, sampled=True), n_per_head=16)
    ref = oracle.attn_rows(Q, K, V, 1.0 / math.sqrt(d), rows)
    offs = oracle.dest_offsets(rows, B, S, H, d, P, rank)
    assert_close(bits_to_f64(got[offs[:, None] + np.arange(d)[None, :]]), ref,
                 "split sweep %r" % ((B, S, H, P, rank, d),))
