"""Pins of the fp64 MoE oracle (CPU only), independent of its own arithmetic:

* the hand-worked example of tests/golden/moe_worked_example.txt (values
  worked on paper from textbook logistic values; fixes the gate/up order,
  SiLU, the W2 orientation, the routing weight, the slot and region);
* SiLU at known points and its identity SiLU(z) - SiLU(-z) = z;
* the all-ranks composition: summing every rank's combine buffer over the k
  slots equals the MoE layer written densely as sum_e G[t, e] FFN_e(x_t) with
  a dense gate matrix G, computed by a separate loop over all experts;
* linearity in the routing weights and in W2, zero gate or up weights;
* ownership: over all ranks every (p, t, j) slot is served exactly once, by
  the rank holding its expert, and a rank's slots are exactly its experts'.

A mutation test plants plausible slips in a copy of the oracle's source and
checks that each makes one of these pins fail.
"""
import math
import os
import types

import numpy as np
import pytest

import oracle.moe_oracle as mo
from moe_inputs import MOE_WORKLOADS, MoeWorkload, moe_rank_weights, moe_tensors
from ua_inputs import to_bf16_bits

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "moe_worked_example.txt")
ORACLE_SRC = os.path.join(os.path.dirname(HERE), "oracle", "moe_oracle.py")


def _golden():
    vals, slots = {}, []
    for line in open(GOLDEN):
        line = line.split("#")[0].split()
        if not line:
            continue
        if line[0] == "slot":
            slots.append((int(line[1]), int(line[2]), int(line[3]), int(line[4]),
                          float(line[5]), float(line[6])))
        else:
            vals[line[0]] = [float(v) for v in line[1:]]
    g = {k: int(v[0]) for k, v in vals.items() if k in ("P", "T", "k", "E", "hidden", "inter")}
    P, T, k, hid, inter = g["P"], g["T"], g["k"], g["hidden"], g["inter"]
    x = to_bf16_bits(np.array(vals["x"], np.float32).reshape(P, T, hid))
    idx = np.array(vals["topk_idx"], np.int32).reshape(P, T, k)
    w = np.array(vals["topk_w"], np.float32).reshape(P, T, k)
    W1 = [to_bf16_bits(np.array(vals["W1_expert%d" % e], np.float32).reshape(2 * inter, hid)) for e in range(g["E"])]
    W2 = [to_bf16_bits(np.array(vals["W2_expert%d" % e], np.float32).reshape(hid, inter)) for e in range(g["E"])]
    return g, x, idx, w, W1, W2, slots


def _check_golden(m):
    g, x, idx, w, W1, W2, slots = _golden()
    P, E = g["P"], g["E"]
    E_l = E // P
    for rank in range(P):
        W1r = np.stack(W1[rank * E_l:(rank + 1) * E_l])
        W2r = np.stack(W2[rank * E_l:(rank + 1) * E_l])
        buf = m.combine_buffer(x, idx, w, W1r, W2r, rank, P, E)
        mine = [s for s in slots if s[0] == rank]
        assert np.count_nonzero(~np.isnan(buf[..., 0])) == len(mine)
        for _, p, t, j, v0, v1 in mine:
            np.testing.assert_allclose(buf[p, t, j], [v0, v1], rtol=1e-14, atol=1e-300)


def test_hand_worked_example():
    _check_golden(mo)


def test_silu_known_points_and_identity():
    assert mo.silu(0.0) == 0.0
    assert abs(mo.silu(1.0) - 0.7310585786300049) < 1e-15
    assert abs(mo.silu(-1.0) + 0.2689414213699951) < 1e-15
    z = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(mo.silu(z) - mo.silu(-z), z, rtol=0, atol=1e-12)
    # large arguments: SiLU(z) -> z and SiLU(-z) -> 0
    assert abs(mo.silu(40.0) - 40.0) < 1e-12 and abs(mo.silu(-40.0)) < 1e-15


def _dense_layer(x_bits, topk_idx, topk_w, W1_all, W2_all):
    """The MoE layer written densely: every expert on every token, weighted by
    a dense gate matrix G[t, e] (zero where e was not chosen)."""
    P, T, k = topk_idx.shape
    E = len(W1_all)
    X = mo.widen(x_bits).reshape(P * T, -1)
    G = np.zeros((P * T, E))
    for n, (idx, w) in enumerate(zip(topk_idx.reshape(-1, k), topk_w.reshape(-1, k))):
        for e, g in zip(idx, w):
            G[n, e] += g
    out = np.zeros_like(X)
    inter = W1_all[0].shape[0] // 2
    for e in range(E):
        W1, W2 = mo.widen(W1_all[e]), mo.widen(W2_all[e])
        for n in range(P * T):
            if G[n, e] == 0.0:
                continue
            gate = W1[:inter] @ X[n]
            up = W1[inter:] @ X[n]
            act = np.array([gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(gate, up)])
            out[n] += G[n, e] * (W2 @ act)
    return out.reshape(P, T, -1)


@pytest.mark.parametrize("routing", ["balanced", "skewed"])
def test_all_ranks_compose_to_the_dense_moe_layer(routing):
    w = MoeWorkload("pin", P=3, rank=0, T=12, hidden=16, inter=8, E=6, k=2, seed=77, routing=routing)
    x, idx, tw, _, _ = moe_tensors(w)
    total = np.zeros((w.P, w.T, w.hidden))
    seen = np.zeros((w.P, w.T, w.k), int)
    W1_all, W2_all = [], []
    for r in range(w.P):
        W1, W2 = moe_rank_weights(w, r)
        W1_all += list(W1)
        W2_all += list(W2)
        buf = mo.combine_buffer(x, idx, tw, W1, W2, r, w.P, w.E)
        own = ~np.isnan(buf[..., 0])
        seen += own
        total += np.where(own[..., None], buf, 0.0).sum(axis=2)
    assert np.all(seen == 1)                                   # every slot served exactly once
    np.testing.assert_allclose(total, _dense_layer(x, idx, tw, W1_all, W2_all), rtol=1e-11, atol=1e-13)


def test_rank_slots_are_exactly_the_ranks_experts():
    w = MOE_WORKLOADS["moe_tiny"]
    x, idx, tw, W1, W2 = moe_tensors(w)
    for r in range(w.P):
        s = mo.rank_slots(idx, r, w.P, w.E)
        e, p, t, j = s.T
        assert np.all(idx[p, t, j] == r * w.E_l + e)
        assert len(s) == np.count_nonzero((idx >= r * w.E_l) & (idx < (r + 1) * w.E_l))
        assert len({tuple(v) for v in s[:, 1:]}) == len(s)
        # ordered by expert, then source rank, token, choice
        assert np.all(np.diff(s[:, 0] * 1e9 + (s[:, 1] * w.T + s[:, 2]) * w.k + s[:, 3]) > 0)


def test_linear_in_routing_weights_and_in_w2_zero_gate_or_up():
    w = MOE_WORKLOADS["moe_tiny"]
    x, idx, tw, W1, W2 = moe_tensors(w)
    base = mo.combine_buffer(x, idx, tw, W1, W2, w.rank, w.P, w.E)
    own = ~np.isnan(base)
    b2 = mo.combine_buffer(x, idx, 2 * tw, W1, W2, w.rank, w.P, w.E)
    np.testing.assert_allclose(b2[own], 2 * base[own], rtol=1e-13, atol=0)
    W2x2 = to_bf16_bits(2 * mo.widen(W2).astype(np.float32))   # exact: a power of two
    b3 = mo.combine_buffer(x, idx, tw, W1, W2x2, w.rank, w.P, w.E)
    np.testing.assert_allclose(b3[own], 2 * base[own], rtol=1e-13, atol=0)
    for half in (0, 1):                                        # zero gate rows / zero up rows
        Wz = W1.copy()
        Wz[:, half * w.inter:(half + 1) * w.inter] = 0
        bz = mo.combine_buffer(x, idx, tw, Wz, W2, w.rank, w.P, w.E)
        assert np.all(bz[own] == 0)


# ---- mutation test: every slip below must make a pin fail ----

MUTANTS = {
    "gate and up swapped": ("a = silu(h[:, :inter]) * h[:, inter:]", "a = silu(h[:, inter:]) * h[:, :inter]"),
    "sigmoid instead of SiLU": ("return z / (1.0 + np.exp(-z))", "return 1.0 / (1.0 + np.exp(-z))"),
    "routing weight dropped": ("out[sel] = topk_w[p, t, j].astype(np.float64)[:, None] * y", "out[sel] = y"),
    "weight of the wrong choice": ("out[sel] = topk_w[p, t, j].astype(np.float64)[:, None] * y",
                                   "out[sel] = topk_w[p, t, 0].astype(np.float64)[:, None] * y"),
    "slot of the wrong choice": ("out[slots[:, 1], slots[:, 2], slots[:, 3]] = vals",
                                 "out[slots[:, 1], slots[:, 2], 0] = vals"),
    "experts strided over ranks": ("np.nonzero(topk_idx == rank * E_l + e)", "np.nonzero(topk_idx == e * P + rank)"),
    "W1 of the neighbouring expert": ("y = expert_ffn(widen(x_bits[p, t]), widen(W1_bits[e]), widen(W2_bits[e]))",
                                      "y = expert_ffn(widen(x_bits[p, t]), widen(W1_bits[(e + 1) % len(W1_bits)]), widen(W2_bits[e]))"),
    "token of the wrong rank": ("y = expert_ffn(widen(x_bits[p, t]),", "y = expert_ffn(widen(x_bits[(p + 1) % x_bits.shape[0], t]),"),
}


def _mutant(old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, old
    m = types.ModuleType("moe_oracle_mutant")
    exec(compile(src.replace(old, new), "moe_oracle_mutant", "exec"), m.__dict__)
    return m


def _pins_fail(m):
    checks = [lambda: _check_golden(m)]

    def compose():
        w = MoeWorkload("pin", P=3, rank=0, T=8, hidden=8, inter=4, E=6, k=2, seed=78)
        x, idx, tw, _, _ = moe_tensors(w)
        total = np.zeros((w.P, w.T, w.hidden))
        W1_all, W2_all = [], []
        for r in range(w.P):
            W1, W2 = moe_rank_weights(w, r)
            W1_all += list(W1)
            W2_all += list(W2)
            buf = m.combine_buffer(x, idx, tw, W1, W2, r, w.P, w.E)
            total += np.nan_to_num(buf).sum(axis=2)
        np.testing.assert_allclose(total, _dense_layer(x, idx, tw, W1_all, W2_all), rtol=1e-11, atol=1e-13)
    checks.append(compose)
    for c in checks:
        try:
            c()
        except Exception:
            return True
    return False


def test_unmodified_oracle_passes_the_pins():
    assert not _pins_fail(mo)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_each_slip_fails_a_pin(name):
    old, new = MUTANTS[name]
    assert _pins_fail(_mutant(old, new)), name
