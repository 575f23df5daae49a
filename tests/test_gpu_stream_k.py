"""GPU parity of the stream-K form of the key split (the *_ws calls where
ua_stream_k_iters > 0): one workgroup per CU, each on an equal run of
(query tile, key tile) iterations across query-tile boundaries, so a
workgroup may finish one query tile's last keys and start the next one's,
and a query tile's keys are cut into up to ua_key_split parts of any length
(down to a single key tile).

Each case asserts the plan is stream-K, then checks (through the key-split
checker) the oracle on sampled rows, the layout, attn_serial_ws +
a2a_permute writing exactly the fused bytes, a second call on the same
workspace bit-equal, and the arrival counts back at zero.
"""
import os

import numpy as np
import pytest

import comm_fusion_amd as ua
from test_gpu_key_split import _check_split_call
from ua_inputs import Workload, make_qkv, sampled_rows

pytestmark = pytest.mark.gpu

# B, S, H, P, rank, d, seed: iterations per workgroup / parts per query tile
SK_CASES = [
    (1, 16384, 40, 8, 7, 128, 61),   # the video heads at 16384 keys: 320 / 2
    (2, 3000, 48, 8, 4, 64, 62),     # d = 64 one row block, ragged last key tile, B = 2: 27 / 3, 1-tile parts
    (1, 5000, 64, 8, 1, 64, 63),     # 50 / 3
    (1, 12344, 24, 8, 6, 128, 64),   # ragged (last key tile 56 keys, last query tile 56 rows): 111 / 3
]


@pytest.mark.parametrize("B,S,H,P,rank,d,seed", SK_CASES)
def test_stream_k_matches_oracle_and_serial(B, S, H, P, rank, d, seed):
    print("stream-K case", (B, S, H, P, rank, d, seed), flush=True)
    assert ua.stream_k_iters(B, S, H, d, P) > 0 and ua.key_split(B, S, H, d, P) >= 2
    Q, K, V = make_qkv(B, S, H // P, d, seed)
    w = Workload("t", B, S, H, P, rank, d, seed, sampled=True)
    _check_split_call(Q, K, V, H, P, rank, sampled_rows(w, n_per_head=64), "stream-K %s" % ((B, S, H, d),))


def stream_k_sweep_shapes(n=12, seed=2030):
    """Random valid shapes on which the plan picks stream-K (the choice is a
    host computation for the full MI355X): B 1-2, P in {1, 2, 4, 8} and any
    rank, 1-8 local heads, both head dims, 2000-20000 keys, mostly ragged;
    at most 3e7 elements per input."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        d = int(rng.choice([64, 128]))
        P = int(rng.choice([1, 2, 4, 8]))
        Hl = int(rng.integers(1, 9))
        B = int(rng.integers(1, 3))
        S = P * int(rng.integers(max(1, 2000 // P), 1 + 20000 // P))
        if B * S * Hl * d > 3e7 or ua.stream_k_iters(B, S, Hl * P, d, P) <= 0:
            continue
        out.append((B, S, Hl * P, P, int(rng.integers(0, P)), d, 800 + len(out)))
    return out


SWEEP = stream_k_sweep_shapes(48, 9105) if os.environ.get("UA_SWEEP_WIDE") == "1" else stream_k_sweep_shapes()


@pytest.mark.parametrize("B,S,H,P,rank,d,seed", SWEEP)
def test_stream_k_sweep(B, S, H, P, rank, d, seed):
    # UA_SWEEP_WIDE=1 draws 48 shapes from another seed instead of 12
    print("stream-K sweep case", (B, S, H, P, rank, d, seed), flush=True)
    Q, K, V = make_qkv(B, S, H // P, d, seed)
    w = Workload("t", B, S, H, P, rank, d, seed, sampled=True)
    _check_split_call(Q, K, V, H, P, rank, sampled_rows(w, n_per_head=32), "stream-K sweep %s" % ((B, S, H, d),))
