"""Seeded sweep of random valid MoE shapes through every form of the expert
path (GPU).

Shapes are drawn once from a fixed seed: P in {1, 2, 3, 4, 8} and any rank,
1-8 local experts, k up to 4 (at most E), 1-300 tokens per rank, hidden a
multiple of 256 up to 1024, intermediate a multiple of 128 up to 384, balanced
or skewed routing (so experts with no rows, one row, and ragged token tiles
come up).  Each shape is checked against the fp64 oracle on every served
Combine slot with the layout exact (test_gpu_moe's tolerance), and the other
forms must write the same bytes: the other schedule, another wave size, the
persistent form (one launch, device tile queue) and the serial form
(experts, then the scatter).  UA_SWEEP_WIDE=1 in the environment draws 80
shapes from another seed instead.
"""
import os

import numpy as np
import pytest

import comm_fusion_amd as ua
from moe_inputs import MOE_SENTINEL_BITS, MoeWorkload
from test_gpu_moe import Case, _check_all, _host_bits, _sentinel

pytestmark = pytest.mark.gpu


def moe_sweep_shapes(n=16, seed=2029):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        P = int(rng.choice([1, 2, 3, 4, 8]))
        E_l = int(rng.integers(1, 9))
        E = P * E_l
        k = int(rng.integers(1, 1 + min(E, 4)))
        T = int(rng.integers(1, 301))
        hidden = 256 * int(rng.integers(1, 5))
        inter = 128 * int(rng.integers(1, 4))
        # the oracle's work on this rank's rows stays small
        if P * T * k * hidden * inter > 2e9:
            continue
        routing = "skewed" if len(out) % 2 else "balanced"
        out.append(MoeWorkload("moe_sweep%d" % len(out), P=P, rank=int(rng.integers(0, P)), T=T, hidden=hidden,
                               inter=inter, E=E, k=k, seed=700 + len(out), routing=routing))
    return out


SHAPES = moe_sweep_shapes(80, 9104) if os.environ.get("UA_SWEEP_WIDE") == "1" else moe_sweep_shapes()


@pytest.mark.parametrize("w", SHAPES, ids=[s.name for s in SHAPES])
def test_moe_sweep(w):
    import torch
    c = Case(w)
    print("moe sweep", w, "N=%d" % c.N, flush=True)
    rng = np.random.default_rng(w.seed + 50)
    g1, g2 = int(rng.integers(1, w.E_l + 1)), int(rng.integers(1, w.E_l + 1))
    ref = _host_bits(c.fused(ua.MOE_INTERLEAVED, g1))
    if c.N:
        _check_all(c, ref, "%s interleaved G %d" % (w.name, g1))
    else:
        assert np.all(ref == MOE_SENTINEL_BITS)   # no row routed here: nothing written
    np.testing.assert_array_equal(_host_bits(c.fused(ua.MOE_EXPERT_WAVE, g2)), ref)
    n_ws = ua.moe_workspace_bytes(w.P, w.T, w.hidden, w.inter, w.E, w.k)
    ws = torch.full((n_ws,), 0xA5, dtype=torch.uint8, device="cuda")
    for schedule, G in ((ua.MOE_INTERLEAVED, g2), (ua.MOE_EXPERT_WAVE, g1)):
        out = _sentinel(c.n_out)
        ua.moe_experts_combine_ws(c.dx, c.drs, c.dtw, c.off, c.dW1, c.dW2, w.P, w.E, out, c.act, ws,
                                  schedule=schedule, experts_per_wave=G)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_host_bits(out), ref)
        if c.N:
            assert int(ws.view(torch.int32)[32]) == 0
    np.testing.assert_array_equal(_host_bits(c.serial(g1)), ref)
