"""Input generator determinism / rounding, and the Burst-Gap relations pinned
against the values printed on the review page of the X-Stage paper (CPU only)."""
import math
import os

import numpy as np
import torch

from oracle import burst_gap
from ua_inputs import WORKLOADS, make_qkv, sampled_rows, to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "xstage_ledger.txt")


def test_same_seed_same_bits_and_different_seeds_differ():
    a = make_qkv(1, 64, 2, 32, 7)
    b = make_qkv(1, 64, 2, 32, 7)
    c = make_qkv(1, 64, 2, 32, 8)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a[0], c[0])


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -1.00390625, 0.0, -0.0], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(to_bf16_bits(x), want)


def test_peaky_keys_are_scaled_within_range():
    q0, k0, v0 = make_qkv(1, 4096, 2, 16, 2, peaky_k=False)
    q1, k1, v1 = make_qkv(1, 4096, 2, 16, 2, peaky_k=True)
    np.testing.assert_array_equal(q0, q1)
    np.testing.assert_array_equal(v0, v1)
    f0 = (k0.astype(np.uint32) << 16).view(np.float32)
    f1 = (k1.astype(np.uint32) << 16).view(np.float32)
    ratio = np.linalg.norm(f1, axis=-1) / np.linalg.norm(f0, axis=-1)
    assert ratio.min() > 0.49 and ratio.max() < 2.01


def test_sampled_rows_include_boundaries_and_are_distinct():
    w = WORKLOADS["video_dit"]
    rows = sampled_rows(w)
    chunk = w.S // w.P
    for h in range(w.Hl):
        s = rows[rows[:, 1] == h][:, 2]
        assert len(np.unique(s)) == len(s) >= 256
        for p in range(1, w.P):
            assert p * chunk - 1 in s and p * chunk in s
        assert 0 in s and w.S - 1 in s
    assert np.array_equal(rows, sampled_rows(w))


def test_workload_sizes():
    w = WORKLOADS["video_dit"]
    assert w.Hl == 5 and w.flops == 4 * 65536 ** 2 * 128 * 5
    assert WORKLOADS["mixed"].out_bytes == 2 * 32768 * 6 * 64 * 2


def _ledger():
    vals = {}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split("=")
            vals[k.strip()] = float(v)
    return vals


def test_burst_gap_relations_reproduce_printed_values():
    g = _ledger()
    MiB = 1024.0 ** 2
    R = g["drain_rate_R_GBps"] * 1e9
    T0 = g["issue_floor_T0_us"] * 1e-6
    # One output tile per producer: Br=128 rows x d=128 bf16 = 32 KiB, K=148.
    tile = 128 * 128 * 2
    assert tile == g["tile_bytes_B_KB"] * 1024
    V = g["producers_K"] * tile
    assert abs(V / MiB - g["burst_V_MiB"]) < 0.05
    backlog = burst_gap.single_burst_backlog(V, R, T0)
    assert abs(backlog / MiB - g["backlog_MiB"]) < 0.05
    assert abs((g["capacity_Q_MiB"] * MiB - backlog) / MiB - g["margin_MiB"]) < 0.01
    m_ub = burst_gap.convergence_seq_len(V, R, T0, g["sigma_us_per_kv_tile"] * 1e-6, 128)
    assert abs(m_ub - g["convergence_M_ub"]) < 50
    # Max law: a gap at least the recovery gap leaves only the floor.
    gstar = burst_gap.recovery_gap(V, R, T0)
    assert math.isclose(burst_gap.issue_time(V, gstar, R, T0), T0)
    assert burst_gap.issue_time(V, 0.0, R, T0) == V / R
    assert burst_gap.rate_bound_ok(V, gstar * 1.001, R, T0)  # V/(T0+G*) = R at equality
    assert not burst_gap.rate_bound_ok(V, 0.0, R, T0 * 0.5)
