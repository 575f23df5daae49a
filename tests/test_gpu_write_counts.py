"""GPU write check of the fused path: every 16-byte chunk of this rank's head
slots in the destination is stored exactly once per call, and nothing outside
them is stored (ua_fused_write_counts counts the epilogue's stores).

The cases cover each launch form: the plain call (one workgroup per query
tile), the equal key split with key groups and with two row blocks per wave,
and the stream-K split whose workgroups cross query-tile boundaries, where a
query tile's parts are merged by whichever part arrives last; ragged tails
and B = 2 among them; the video and long-DiT workloads at full size.  The
counted call's output must also be bit-equal to the product call's.
"""
import numpy as np
import pytest

import comm_fusion_amd as ua
from gpu_helpers import sentinel_buffer, to_dev, to_host_bits
from ua_inputs import make_qkv

pytestmark = pytest.mark.gpu

# B, S, H, P, rank, d, seed, form: "plain", "split" (equal runs) or "stream-k"
CASES = [
    (1, 65536, 40, 8, 7, 128, 71, "plain"),    # the video workload, full size
    (2, 32768, 24, 4, 1, 64, 72, "plain"),     # d = 64, B = 2
    (1, 304, 8, 2, 1, 64, 73, "plain"),        # ragged single query tile per head
    (1, 4096, 24, 8, 3, 128, 74, "split"),     # two key groups, 2 parts
    (1, 16384, 48, 8, 1, 64, 75, "split"),     # two row blocks per wave, 4 parts
    (1, 8176, 8, 8, 2, 128, 76, "split"),      # ragged query and key tails, 4 parts
    (2, 1000, 16, 4, 3, 128, 77, "split"),     # ragged, B = 2
    (1, 16384, 24, 8, 5, 128, 78, "stream-k"),  # the long-DiT workload, full size
    (2, 3000, 48, 8, 4, 64, 79, "stream-k"),   # parts down to one key tile, B = 2
]


def _form(B, S, H, d, P):
    if ua.key_split(B, S, H, d, P) <= 1:
        return "plain"
    return "stream-k" if ua.stream_k_iters(B, S, H, d, P) > 0 else "split"


@pytest.mark.parametrize("B,S,H,P,rank,d,seed,form", CASES)
def test_each_owned_chunk_is_written_once(B, S, H, P, rank, d, seed, form):
    import torch
    print("write-count case", (B, S, H, P, rank, d, seed, form), flush=True)
    assert _form(B, S, H, d, P) == form
    Hl = H // P
    Q, K, V = make_qkv(B, S, Hl, d, seed)
    q, k, v = (to_dev(x).view(*x.shape) for x in (Q, K, V))
    ws = ua.new_workspace(B, S, H, d, P, q.device)
    n = B * S * H * d
    out = sentinel_buffer(n)
    counts = torch.zeros(n // 8, dtype=torch.int32, device="cuda")
    ua.fused_write_counts(q, k, v, rank, P, out, counts, workspace=ws)
    ref = sentinel_buffer(n)
    if ws is None:
        ua.attn_ulysses_fused(q, k, v, rank, P, ref)
    else:
        ua.attn_ulysses_fused_ws(q, k, v, rank, P, ref, ws)
    torch.cuda.synchronize()
    c = counts.view(B, S, H, d // 8)
    own = c[:, :, rank * Hl:(rank + 1) * Hl]
    assert int(own.min()) == 1 and int(own.max()) == 1, \
        "owned chunks written %d..%d times" % (int(own.min()), int(own.max()))
    assert int(c.sum()) == B * S * Hl * (d // 8), "a chunk outside this rank's heads was written"
    np.testing.assert_array_equal(to_host_bits(out), to_host_bits(ref))
