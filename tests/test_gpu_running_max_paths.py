"""GPU parity of the softmax's exact path in every launch form.

The steady loop takes P against the running max as it stands and sends a key
tile to an exact path (its scores formed again from K in global memory, the
max raised, P formed again) when a lane's sum of the tile's P passes 2^15.
These cases put such tiles in the middle of the calls that the running-max
test of the plain call does not reach: the equal key split (key groups), the
stream-K split (parts cut at workgroup boundaries), and the call that reads Q,
K, V in place from the sequence-partitioned inputs (row stride H*d, which the
exact path's global K reads use too).  Key rows are scaled so that the
running max keeps rising along the keys, or jumps at three keys inside the
parts; each case is checked against the oracle on sampled rows, the layout,
the serial form and a second call on the same workspace (through the
key-split checker), and the io call bit-equal to gather + fused.
"""
import math

import numpy as np
import pytest

import comm_fusion_amd as ua
import oracle
from gpu_helpers import bits_to_f64, check_dest_layout, sentinel_buffer, to_dev, to_host_bits
from test_gpu_key_split import _check_split_call
from test_gpu_parity import _compare_rows, _fused
from ua_inputs import Workload, make_qkv, sampled_rows, to_bf16_bits

pytestmark = pytest.mark.gpu


def _shaped_k(K, S, pattern, spikes):
    Kf = bits_to_f64(K)
    if pattern == "rising":
        Kf *= (0.25 + 3.0 * np.arange(S) / S)[None, :, None, None]
    else:
        for j in spikes:
            Kf[:, j] *= 60.0
    return to_bf16_bits(Kf.astype(np.float32))


# B, S, H, P, rank, d, seed, form
SPLIT_CASES = [
    (1, 4096, 24, 8, 3, 128, 91, "split"),     # two key groups, 2-way split
    (1, 16384, 24, 8, 5, 128, 92, "stream-k"),  # stream-K, 192 iterations per workgroup
    (2, 3000, 48, 8, 4, 64, 93, "stream-k"),   # stream-K with one-tile parts, d = 64
]


@pytest.mark.parametrize("B,S,H,P,rank,d,seed,form", SPLIT_CASES)
@pytest.mark.parametrize("pattern", ["rising", "spikes"])
def test_exact_path_inside_split_calls(B, S, H, P, rank, d, seed, form, pattern):
    print("exact-path case", (B, S, H, P, rank, d, seed, form, pattern), flush=True)
    sk = ua.stream_k_iters(B, S, H, d, P)
    assert ua.key_split(B, S, H, d, P) >= 2 and (sk > 0) == (form == "stream-k")
    Q, K, V = make_qkv(B, S, H // P, d, seed)
    K = _shaped_k(K, S, pattern, (S // 3, S // 2 + 7, (2 * S) // 3 + 33))
    w = Workload("t", B, S, H, P, rank, d, seed, sampled=True)
    _check_split_call(Q, K, V, H, P, rank, sampled_rows(w, n_per_head=64), "%s %s" % (form, pattern))


@pytest.mark.parametrize("pattern", ["rising", "spikes"])
def test_exact_path_with_inputs_read_in_place(pattern):
    B, S, H, P, rank, d, seed = 1, 2048, 16, 4, 2, 128, 94
    print("exact-path io case", pattern, flush=True)
    Hl = H // P
    # sequence-partitioned projections [B][S][H][d]; this rank's heads are
    # columns rank*Hl .. rank*Hl + Hl - 1
    Xq, Xk, Xv = make_qkv(B, S, H, d, seed)
    Xk = _shaped_k(Xk, S, pattern, (300, 1023, 1500))
    io = sentinel_buffer(B * S * H * d)
    ua.attn_ulysses_fused_io(to_dev(Xq).view(*Xq.shape), to_dev(Xk).view(*Xk.shape), to_dev(Xv).view(*Xv.shape),
                             rank, P, io)
    import torch
    torch.cuda.synchronize()
    got = to_host_bits(io)
    G = [oracle.gather(x, H, P, rank) for x in (Xq, Xk, Xv)]
    np.testing.assert_array_equal(got, _fused(*G, rank, P, H))
    check_dest_layout(got, B, S, H, d, P, rank)
    rows = sampled_rows(Workload("t", B, S, H, P, rank, d, seed, sampled=True), n_per_head=96)
    _compare_rows(got, *G, rows, H, P, rank, 1.0 / math.sqrt(d), "io " + pattern)
