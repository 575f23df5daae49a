"""Repeated calls of the launches whose workgroups hand results to each
other through device memory: the key-split and stream-K attention calls
(partial results, arrival counts, the merging workgroup's loads) and the
persistent MoE call (the device tile queue, per-token-tile release counts
and the Linear-2 tiles' bounded waits).

Each case runs a few hundred calls back to back on one workspace, with two
inputs alternating, into a ring of output buffers, and requires every output
to equal its input's first result bit for bit.  A merge that read a partial
not yet stored (or one left from the previous call, computed from the other
input), or a Linear-2 tile that read act rows before they were complete,
would show as a differing output; the MoE workspace's count of bounded waits
that gave up must stay zero.  The first results themselves are checked
against the oracle by the parity tests of each form; here they are checked
against the serial call (attention) and the per-wave launches (MoE).
"""
import numpy as np
import pytest

import comm_fusion_amd as ua
from gpu_helpers import sentinel_buffer, to_dev
from moe_inputs import MOE_WORKLOADS
from test_gpu_moe import Case
from ua_inputs import make_qkv

pytestmark = pytest.mark.gpu

RING = 8


def _run_ring(calls, refs, n_calls, what, after=None):
    """calls[j](out) for j alternating over len(calls) inputs; every output
    must equal refs[j] bit for bit."""
    import torch
    n = refs[0].numel()
    outs = [sentinel_buffer(n) for _ in range(RING)]
    done = 0
    while done < n_calls:
        batch = min(RING, n_calls - done)
        for i in range(batch):
            calls[(done + i) % len(calls)](outs[i])
        torch.cuda.synchronize()
        for i in range(batch):
            j = (done + i) % len(calls)
            assert torch.equal(outs[i].view(torch.int16), refs[j].view(torch.int16)), \
                "%s: call %d (input %d) differs from the first result" % (what, done + i, j)
        if after is not None:
            after(done + batch)
        done += batch


# B, S, H, P, rank, d, form
SPLIT_CASES = [
    (1, 16384, 24, 8, 5, 128, "stream-k"),  # the long-DiT workload's shape
    (1, 4096, 24, 8, 3, 128, "split"),      # the DiT-image shape: two key groups, 2 parts
    (2, 3000, 48, 8, 4, 64, "stream-k"),    # parts down to one key tile, d = 64
    (1, 16384, 48, 8, 1, 64, "split"),      # two row blocks per wave, 4 parts
]


@pytest.mark.parametrize("B,S,H,P,rank,d,form", SPLIT_CASES)
def test_split_calls_repeat_bit_identically(B, S, H, P, rank, d, form):
    import torch
    print("repeat case", (B, S, H, P, rank, d, form), flush=True)
    assert ua.key_split(B, S, H, d, P) > 1
    assert (ua.stream_k_iters(B, S, H, d, P) > 0) == (form == "stream-k")
    Hl = H // P
    ws = ua.new_workspace(B, S, H, d, P, "cuda")
    ins, refs = [], []
    for seed in (301, 302):
        q, k, v = (to_dev(x).view(*x.shape) for x in make_qkv(B, S, Hl, d, seed))
        ins.append((q, k, v))
        # the serial call's result, permuted: the reference bytes of the fused call
        loc = torch.empty((B, S, Hl, d), dtype=torch.bfloat16, device="cuda")
        ua.attn_serial_ws(q, k, v, rank, P, loc, ws)
        ref = sentinel_buffer(B * S * H * d)
        ua.a2a_permute(loc, rank, P, ref)
        refs.append(ref)
    torch.cuda.synchronize()
    calls = [lambda out, x=x: ua.attn_ulysses_fused_ws(*x, rank, P, out, ws) for x in ins]
    _run_ring(calls, refs, 256, "split %s" % form)


def test_persistent_moe_calls_repeat_bit_identically():
    import torch
    w = MOE_WORKLOADS["moe_ds"]
    cases = [Case(w)]
    # the other input: the same shapes and routing, other token rows
    x2 = np.ascontiguousarray(cases[0].x[::-1])
    cases.append(Case(w, (x2, cases[0].idx, cases[0].tw, cases[0].W1, cases[0].W2)))
    print("repeat case moe_ds N=%d" % cases[0].N, flush=True)
    n_ws = ua.moe_workspace_bytes(w.P, w.T, w.hidden, w.inter, w.E, w.k)
    ws = torch.full((n_ws,), 0xA5, dtype=torch.uint8, device="cuda")
    # one act buffer shared by both inputs, as a caller reusing its scratch would
    act = cases[0].act
    refs = [c.fused(ua.MOE_INTERLEAVED, 8) for c in cases]

    def call(out, c):
        ua.moe_experts_combine_ws(c.dx, c.drs, c.dtw, c.off, c.dW1, c.dW2, w.P, w.E, out, act, ws,
                                  schedule=ua.MOE_INTERLEAVED, experts_per_wave=8)

    def no_timeouts(n):
        assert int(ws.view(torch.int32)[32]) == 0, "a bounded wait gave up within the first %d calls" % n

    assert not torch.equal(refs[0].view(torch.int16), refs[1].view(torch.int16))
    _run_ring([lambda out, c=c: call(out, c) for c in cases], refs, 96, "persistent moe_ds", after=no_timeouts)
