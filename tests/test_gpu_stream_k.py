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
