"""The entry points inside a captured HIP graph (through torch.cuda.CUDAGraph).

They allocate nothing and issue no memset, so a caller can capture them.
The graph is replayed several times with eager work and synchronisation in
between; every replay is checked bit for bit against the eager calls, and an
input changed between replays must show up in the next replay's output.
"""
import numpy as np
import pytest

import comm_fusion_amd as ua
from gpu_helpers import sentinel_buffer, to_dev
from ua_inputs import SENTINEL_BITS, make_qkv

pytestmark = pytest.mark.gpu


def test_fused_calls_replay_from_a_graph():
    import torch
    B, S, H, P, rank, d = 1, 1032, 96, 3, 2, 128
    Hl = H // P
    Xq, Xk, Xv = (to_dev(x).view(B, S, H, d) for x in make_qkv(B, S, H, d, 30))
    q, k, v = (x[:, :, rank * Hl:(rank + 1) * Hl].contiguous() for x in (Xq, Xk, Xv))
    n = B * S * H * d
    fused, fused_io = sentinel_buffer(n), sentinel_buffer(n)
    gathered = torch.empty_like(q)

    def calls():
        ua.attn_ulysses_fused(q, k, v, rank, P, fused)
        ua.attn_ulysses_fused_io(Xq, Xk, Xv, rank, P, fused_io)
        ua.a2a_gather(Xv, rank, P, gathered)

    calls()
    torch.cuda.synchronize()
    ref_fused, ref_io = fused.clone(), fused_io.clone()
    assert torch.equal(ref_fused.view(torch.int16), ref_io.view(torch.int16))
    assert torch.equal(gathered, v)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()

    sentinel = SENTINEL_BITS - 0x10000 if SENTINEL_BITS >= 0x8000 else SENTINEL_BITS
    for _ in range(3):
        fused.view(torch.int16).fill_(sentinel)
        fused_io.view(torch.int16).fill_(sentinel)
        gathered.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(fused.view(torch.int16), ref_fused.view(torch.int16))
        assert torch.equal(fused_io.view(torch.int16), ref_io.view(torch.int16))
        assert torch.equal(gathered, v)

    # V doubled in place (exact in bf16): attention is linear in V and the
    # weights are unchanged, so the replay must return exactly twice the output
    # in this rank's slots, and the gather the doubled rows.
    v.mul_(2)
    Xv.mul_(2)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    own = fused.view(B, S, H, d)[:, :, rank * Hl:(rank + 1) * Hl]
    ref_own = ref_fused.view(B, S, H, d)[:, :, rank * Hl:(rank + 1) * Hl]
    assert torch.equal(own, ref_own * 2)
    assert torch.equal(fused_io.view(torch.int16), fused.view(torch.int16))
    assert torch.equal(gathered, v)
    others = np.delete(fused.view(torch.int16).view(B, S, H, d).cpu().numpy(),
                       np.s_[rank * Hl:(rank + 1) * Hl], axis=2)
    assert np.all(others.view(np.uint16) == SENTINEL_BITS)


def test_key_split_call_replays_from_a_graph():
    # The workspace's arrival counts are reset by the kernel itself, so every
    # replay (no memset in the graph) returns the eager call's bits.
    import torch
    B, S, H, P, rank, d = 2, 2048, 8, 2, 1, 64
    assert ua.key_split(B, S, H, d, P) > 1
    q, k, v = (to_dev(x).view(B, S, H // P, d) for x in make_qkv(B, S, H // P, d, 31))
    ws = ua.new_workspace(B, S, H, d, P, q.device)
    out = sentinel_buffer(B * S * H * d)
    ua.attn_ulysses_fused_ws(q, k, v, rank, P, out, ws)
    torch.cuda.synchronize()
    ref = out.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ua.attn_ulysses_fused_ws(q, k, v, rank, P, out, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ua.attn_ulysses_fused_ws(q, k, v, rank, P, out, ws)
    sentinel = SENTINEL_BITS - 0x10000 if SENTINEL_BITS >= 0x8000 else SENTINEL_BITS
    for _ in range(3):
        out.view(torch.int16).fill_(sentinel)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_noalloc_call_replays_from_a_graph():
    # The call for callers that cannot allocate: its key-split workspace is
    # the library's fixed scratch, whose arrival counts each call clears with
    # a small kernel (no memset), so it can be captured.  Between replays an
    # eager call of another split shape leaves its own partials and counts
    # in the scratch; every replay must still return the eager call's bits.
    import torch
    B, S, H, P, rank, d = 1, 4096, 24, 8, 3, 128
    assert ua.key_split(B, S, H, d, P) > 1
    q, k, v = (to_dev(x).view(B, S, H // P, d) for x in make_qkv(B, S, H // P, d, 33))
    out = sentinel_buffer(B * S * H * d)
    ua.attn_ulysses_fused_noalloc(q, k, v, rank, P, out)   # first call on the device: set-up, eager
    torch.cuda.synchronize()
    ref = out.clone()
    ws = ua.new_workspace(B, S, H, d, P, q.device)
    via_ws = sentinel_buffer(B * S * H * d)
    ua.attn_ulysses_fused_ws(q, k, v, rank, P, via_ws, ws)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16), via_ws.view(torch.int16))
    # another split shape for the eager calls between replays (d = 64, two row blocks)
    B2, S2, H2, P2, r2, d2 = 1, 16384, 48, 8, 1, 64
    assert ua.key_split(B2, S2, H2, d2, P2) > 1
    q2, k2, v2 = (to_dev(x).view(B2, S2, H2 // P2, d2) for x in make_qkv(B2, S2, H2 // P2, d2, 34))
    out2 = sentinel_buffer(B2 * S2 * H2 * d2)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ua.attn_ulysses_fused_noalloc(q, k, v, rank, P, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ua.attn_ulysses_fused_noalloc(q, k, v, rank, P, out)
    sentinel = SENTINEL_BITS - 0x10000 if SENTINEL_BITS >= 0x8000 else SENTINEL_BITS
    for _ in range(3):
        ua.attn_ulysses_fused_noalloc(q2, k2, v2, r2, P2, out2)
        out.view(torch.int16).fill_(sentinel)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_moe_experts_combine_replays_from_a_graph():
    """The MoE path (several launches per call, both schedules, and the
    persistent form with its workspace clear) inside a graph: every replay
    bit-equal to the eager call, with the workspace refilled with garbage
    between replays; routing weights doubled in place (exact in fp32, and the
    weighted output is rounded once) show up in the next replay."""
    import torch
    from moe_inputs import MOE_SENTINEL_BITS, MOE_WORKLOADS, moe_tensors
    w = MOE_WORKLOADS["moe_small_skewed"]
    x, idx, tw, W1, W2 = moe_tensors(w)
    off, slots = ua.moe_recv_layout(idx, w.rank, w.P, w.hidden, w.inter, w.E)
    N = int(off[-1])
    dx, dW1, dW2 = (to_dev(a) for a in (x, W1, W2))
    dtw = torch.from_numpy(np.ascontiguousarray(tw)).cuda()
    drs = torch.from_numpy(slots.astype(np.int32)).cuda()
    act = torch.empty(N * w.inter, dtype=torch.bfloat16, device="cuda")
    sentinel = MOE_SENTINEL_BITS - 0x10000 if MOE_SENTINEL_BITS >= 0x8000 else MOE_SENTINEL_BITS
    n_out = w.P * w.T * w.k * w.hidden
    outs = [torch.full((n_out,), sentinel, dtype=torch.int16, device="cuda").view(torch.bfloat16) for _ in range(3)]
    ws = ua.new_moe_workspace(dx.view(w.P, w.T, w.hidden), dW1.view(w.E_l, 2 * w.inter, w.hidden), dtw, w.P, w.E)
    ws.fill_(0xA5)

    def calls():
        ua.moe_experts_combine(dx, drs, dtw, off, dW1, dW2, w.P, w.E, outs[0], act,
                               schedule=ua.MOE_INTERLEAVED, experts_per_wave=3)
        ua.moe_experts_combine(dx, drs, dtw, off, dW1, dW2, w.P, w.E, outs[1], act,
                               schedule=ua.MOE_EXPERT_WAVE, experts_per_wave=3)
        ua.moe_experts_combine_ws(dx, drs, dtw, off, dW1, dW2, w.P, w.E, outs[2], act, ws,
                                  schedule=ua.MOE_INTERLEAVED, experts_per_wave=3)

    calls()
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    assert torch.equal(refs[0].view(torch.int16), refs[1].view(torch.int16))
    assert torch.equal(refs[0].view(torch.int16), refs[2].view(torch.int16))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for _ in range(3):
        for o in outs:
            o.view(torch.int16).fill_(sentinel)
        act.zero_()
        ws.fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o.view(torch.int16), r.view(torch.int16))
        assert int(ws.view(torch.int32)[32]) == 0

    dtw.mul_(2)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    served = torch.zeros(w.P * w.T * w.k, dtype=torch.bool, device="cuda")
    served[drs.long()] = True
    got = outs[0].view(-1, w.hidden)[served].float()
    ref = refs[0].view(-1, w.hidden)[served].float()
    assert torch.equal(got, ref * 2)
    assert torch.equal(outs[1].view(torch.int16), outs[0].view(torch.int16))
    assert torch.equal(outs[2].view(torch.int16), outs[0].view(torch.int16))
