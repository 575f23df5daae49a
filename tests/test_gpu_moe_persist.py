"""GPU parity of the MoE path's persistent form (moe_experts_combine_ws,
moe_experts_local_ws): one launch whose workgroups take the schedule's tiles
from a device queue, each Linear-2 tile waiting for the Linear-1 tiles of its
token rows.

Every tile runs the same arithmetic as in the per-wave launches, so each
case requires the persistent output to be bit-identical to
moe_experts_combine's (itself checked against the fp64 oracle in
test_gpu_moe.py), plus the oracle on the small workloads, and the workspace's
count of bounded waits that gave up to stay zero.  Two inputs alternate on one
act buffer and workspace, so a Linear-2 tile that read an act row left from
the previous call (or cached from it) would differ."""
import numpy as np
import pytest

import comm_fusion_amd as ua
from moe_inputs import MOE_WORKLOADS, MoeWorkload, moe_tensors
from test_gpu_moe import Case, _check_all, _host_bits, _sentinel

pytestmark = pytest.mark.gpu

TIMEOUT_WORD = 32


def _persist(c: Case, schedule, G, ws):
    import torch
    out = _sentinel(c.n_out)
    ua.moe_experts_combine_ws(c.dx, c.drs, c.dtw, c.off, c.dW1, c.dW2, c.w.P, c.w.E, out, c.act, ws,
                              schedule=schedule, experts_per_wave=G)
    torch.cuda.synchronize()
    return out


def _timeouts(ws):
    import torch
    return int(ws.view(torch.int32)[TIMEOUT_WORD])


def _ws(c: Case):
    import torch
    n = ua.moe_workspace_bytes(c.w.P, c.w.T, c.w.hidden, c.w.inter, c.w.E, c.w.k)
    # filled with garbage: the call clears what it uses
    return torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("name", ["moe_tiny", "moe_small", "moe_small_skewed"])
def test_persistent_equals_the_launch_form_and_the_oracle(name):
    w = MOE_WORKLOADS[name]
    c = Case(w)
    ws = _ws(c)
    print("moe persistent case %s N=%d" % (name, c.N), flush=True)
    ref = _host_bits(c.fused(ua.MOE_INTERLEAVED, 1))
    _check_all(c, ref, name + " launch form")
    for schedule in (ua.MOE_EXPERT_WAVE, ua.MOE_INTERLEAVED):
        for G in (1, 3, w.E_l):
            got = _host_bits(_persist(c, schedule, G, ws))
            np.testing.assert_array_equal(got, ref, err_msg="%s schedule %d G %d" % (name, schedule, G))
            assert _timeouts(ws) == 0


def test_persistent_local_form_equals_the_launch_form():
    import torch
    w = MOE_WORKLOADS["moe_small_skewed"]
    c = Case(w)
    ws = _ws(c)
    ys = []
    for persist in (False, True):
        y = torch.empty(c.N * w.hidden, dtype=torch.bfloat16, device="cuda")
        if persist:
            ua.moe_experts_local_ws(c.dx, c.drs, c.dtw, c.off, c.dW1, c.dW2, w.P, w.E, y, c.act, ws,
                                    experts_per_wave=2)
        else:
            ua.moe_experts_local(c.dx, c.drs, c.dtw, c.off, c.dW1, c.dW2, w.P, w.E, y, c.act, experts_per_wave=2)
        torch.cuda.synchronize()
        ys.append(_host_bits(y))
    np.testing.assert_array_equal(ys[1], ys[0])
    assert _timeouts(ws) == 0


def test_persistent_ragged_and_empty_experts():
    # the routing of test_gpu_moe.py's ragged case: rows per local expert
    # 0, 1, 127, 128, 129, 300
    w = MoeWorkload("moe_edge", P=2, rank=1, T=400, hidden=256, inter=128, E=12, k=2, seed=31)
    x, _, tw, W1, W2 = moe_tensors(w)
    want = [0, 1, 127, 128, 129, 300]
    rng = np.random.default_rng(5)
    idx = np.zeros((w.P, w.T, w.k), np.int32)
    flat = idx.reshape(-1, w.k)
    pool = rng.permutation(w.P * w.T)
    pos = 0
    for e, n in enumerate(want):
        for t in pool[pos:pos + n]:
            flat[t, 0] = 6 + e
        pos += n
    for t in pool[pos:]:
        flat[t, 0] = rng.integers(0, 6)
    for t in range(len(flat)):
        flat[t, 1] = (flat[t, 0] + 1) % 6 if flat[t, 0] < 6 else rng.integers(0, 6)
    c = Case(w, (x, idx, tw, W1, W2))
    assert list(np.diff(c.off)) == want
    ws = _ws(c)
    ref = _host_bits(c.fused(ua.MOE_INTERLEAVED, 2))
    for schedule, G in ((ua.MOE_INTERLEAVED, 2), (ua.MOE_EXPERT_WAVE, 1), (ua.MOE_INTERLEAVED, 6)):
        np.testing.assert_array_equal(_host_bits(_persist(c, schedule, G, ws)), ref)
    assert _timeouts(ws) == 0


@pytest.mark.parametrize("name", ["moe_ds", "moe_ds_skewed"])
def test_persistent_full_size_alternating_inputs(name):
    import torch
    w = MOE_WORKLOADS[name]
    c = Case(w)
    ws = _ws(c)
    print("moe persistent full size %s N=%d" % (name, c.N), flush=True)
    # a second token buffer (same routing, other values) sharing act and the workspace
    xb = moe_tensors(MoeWorkload(w.name + "_b", w.P, w.rank, w.T, w.hidden, w.inter, w.E, w.k, w.seed + 7,
                                 w.routing))[0]
    xs = {"a": c.dx, "b": torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).cuda()}
    refs = {}
    for key in ("a", "b"):
        c.dx = xs[key]
        refs[key] = c.fused(ua.MOE_INTERLEAVED, 8).view(torch.int16)
    assert not torch.equal(refs["a"], refs["b"])
    calls = (("a", 8, ua.MOE_INTERLEAVED), ("b", 8, ua.MOE_INTERLEAVED), ("a", 4, ua.MOE_EXPERT_WAVE),
             ("b", 32, ua.MOE_INTERLEAVED), ("a", 8, ua.MOE_INTERLEAVED))
    for i, (key, G, sch) in enumerate(calls):
        c.dx = xs[key]
        got = _persist(c, sch, G, ws).view(torch.int16)
        assert torch.equal(got, refs[key]), "call %d: input %s, G %d, schedule %d" % (i, key, G, sch)
        assert _timeouts(ws) == 0


@pytest.mark.parametrize("G", [3, 32])
def test_persistent_form_over_several_launches(G):
    # 80 local experts: at 3 experts per wave a launch holds 10 waves (30
    # experts), at 32 one wave, so the call runs 3 launches, each with its
    # own queue counter in the workspace
    w = MoeWorkload("moe_many", P=2, rank=1, T=512, hidden=256, inter=128, E=160, k=4, seed=41)
    c = Case(w)
    ws = _ws(c)
    print("moe persistent, %d local experts, G %d, N=%d" % (w.E_l, G, c.N), flush=True)
    ref = _host_bits(c.fused(ua.MOE_INTERLEAVED, G))
    _check_all(c, ref, "many experts, launch form")
    for schedule in (ua.MOE_INTERLEAVED, ua.MOE_EXPERT_WAVE):
        np.testing.assert_array_equal(_host_bits(_persist(c, schedule, G, ws)), ref)
        assert _timeouts(ws) == 0
