"""GPU parity of the MoE expert path with the Combine fused into Linear-2
(moe_experts_combine) against the fp64 oracle.

Every case checks, on seeded inputs: the values of every served Combine slot
(or sampled slots at the full DeepSeek-style size) within the tolerance
derived in the design notes; the layout bit-exactly (served slots written,
every other slot keeps the sentinel); the Expert-Wave and interleaved
schedules, at several wave sizes, bit-identical; and the serial form
(moe_experts_local, then moe_combine_scatter) writing exactly the fused bytes.

Tolerance (bf16 outputs against fp64, over all compared elements): max-abs
<= 1e-2 * max|ref| and relative RMS <= 4e-3.  Two bf16 roundings set the
expected error: the activation between the layers and the output, each a
uniform error over an ulp of 2^-8 to 2^-7 of the value, ~1.6e-3 relative
RMS; together ~2.3e-3 (measured: 2.35e-3 on every case, max-abs <= 0.5% of
max|ref|).
"""
import numpy as np
import pytest

import comm_fusion_amd as ua
import oracle.moe_oracle as mo
from moe_inputs import MOE_SENTINEL_BITS, MOE_WORKLOADS, MoeWorkload, moe_tensors

pytestmark = pytest.mark.gpu

MAX_ABS_REL = 1e-2
REL_RMS = 4e-3


def _bits_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _sentinel(n):
    import torch
    return torch.full((n,), MOE_SENTINEL_BITS, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def _host_bits(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _f64(bits):
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _assert_close(got, ref, what):
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    err = np.abs(got - ref)
    scale = max(np.abs(ref).max(), 1e-30)
    rel_rms = np.sqrt((err ** 2).sum() / max((ref ** 2).sum(), 1e-300))
    msg = "%s: max-abs %.3g (%.3g of max|ref|), rel-RMS %.3g" % (what, err.max(), err.max() / scale, rel_rms)
    print(msg, flush=True)
    assert err.max() <= MAX_ABS_REL * scale and rel_rms <= REL_RMS, msg
    return err.max() / scale, rel_rms


class Case:
    def __init__(self, w: MoeWorkload, tensors=None):
        import torch
        self.w = w
        self.x, self.idx, self.tw, self.W1, self.W2 = tensors or moe_tensors(w)
        self.off, self.slots = ua.moe_recv_layout(self.idx, w.rank, w.P, w.hidden, w.inter, w.E)
        self.N = int(self.off[-1])
        self.dx = _bits_dev(self.x)
        self.dW1 = _bits_dev(self.W1)
        self.dW2 = _bits_dev(self.W2)
        self.dtw = torch.from_numpy(np.ascontiguousarray(self.tw)).cuda()
        self.drs = torch.from_numpy(self.slots.astype(np.int32)).cuda()
        self.act = torch.empty(max(self.N, 1) * w.inter, dtype=torch.bfloat16, device="cuda")[: self.N * w.inter]
        self.n_out = w.P * w.T * w.k * w.hidden

    def fused(self, schedule, G):
        import torch
        out = _sentinel(self.n_out)
        ua.moe_experts_combine(self.dx, self.drs, self.dtw, self.off, self.dW1, self.dW2, self.w.P, self.w.E,
                               out, self.act, schedule=schedule, experts_per_wave=G)
        torch.cuda.synchronize()
        return out

    def serial(self, G):
        import torch
        w = self.w
        y = torch.empty(self.N * w.hidden, dtype=torch.bfloat16, device="cuda")
        ua.moe_experts_local(self.dx, self.drs, self.dtw, self.off, self.dW1, self.dW2, w.P, w.E, y, self.act,
                             experts_per_wave=G)
        out = _sentinel(self.n_out)
        ua.moe_combine_scatter(y, self.drs, self.N, w.P, w.T, w.hidden, w.inter, w.E, w.k, out)
        torch.cuda.synchronize()
        return out


def _check_layout(bits, c: Case):
    w = c.w
    rows = bits.reshape(w.P * w.T * w.k, w.hidden)
    served = np.zeros(len(rows), bool)
    served[c.slots] = True
    assert np.all(rows[~served] == MOE_SENTINEL_BITS), "a slot not served here was written"
    assert not np.any(rows[served] == MOE_SENTINEL_BITS), "a served slot keeps the sentinel"


def _check_all(c: Case, bits, what):
    w = c.w
    ref = mo.combine_buffer(c.x, c.idx, c.tw, c.W1, c.W2, w.rank, w.P, w.E).reshape(-1, w.hidden)
    got = _f64(bits).reshape(-1, w.hidden)
    _check_layout(bits, c)
    return _assert_close(got[c.slots], ref[c.slots], what)


@pytest.mark.parametrize("name", ["moe_tiny", "moe_small", "moe_small_skewed"])
def test_schedules_match_the_oracle_and_each_other(name):
    w = MOE_WORKLOADS[name]
    c = Case(w)
    print("moe case %s N=%d" % (name, c.N), flush=True)
    ref_bits = None
    for schedule in (ua.MOE_EXPERT_WAVE, ua.MOE_INTERLEAVED):
        for G in (1, 3, w.E_l):
            bits = _host_bits(c.fused(schedule, G))
            if ref_bits is None:
                _check_all(c, bits, "%s schedule %d G %d" % (name, schedule, G))
                ref_bits = bits
            else:
                np.testing.assert_array_equal(bits, ref_bits)
    np.testing.assert_array_equal(_host_bits(c.serial(2)), ref_bits)


def test_ragged_and_empty_experts():
    # rows per local expert 0, 1, 127, 128, 129 and 300: ragged token tiles,
    # an expert with no rows, one with a single row
    w = MoeWorkload("moe_edge", P=2, rank=1, T=400, hidden=256, inter=128, E=12, k=2, seed=31)
    x, _, tw, W1, W2 = moe_tensors(w)
    want = [0, 1, 127, 128, 129, 300]          # rows of rank 1's experts 6..11
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
        flat[t, 0] = rng.integers(0, 6)          # a rank-0 expert
    for t in range(len(flat)):                   # second choice: a rank-0 expert
        flat[t, 1] = (flat[t, 0] + 1) % 6 if flat[t, 0] < 6 else rng.integers(0, 6)
    c = Case(w, (x, idx, tw, W1, W2))
    assert list(np.diff(c.off)) == want
    bits = _host_bits(c.fused(ua.MOE_INTERLEAVED, 2))
    _check_all(c, bits, "ragged")
    np.testing.assert_array_equal(_host_bits(c.fused(ua.MOE_EXPERT_WAVE, 1)), bits)
    np.testing.assert_array_equal(_host_bits(c.serial(6)), bits)


def test_no_rows_routed_here_writes_nothing():
    w = MoeWorkload("moe_none", P=2, rank=1, T=16, hidden=256, inter=128, E=4, k=1, seed=32)
    x, idx, tw, W1, W2 = moe_tensors(w)
    idx[:] = 0                                    # every token chose an expert of rank 0
    c = Case(w, (x, idx, tw, W1, W2))
    assert c.N == 0
    bits = _host_bits(c.fused(ua.MOE_INTERLEAVED, 1))
    assert np.all(bits == MOE_SENTINEL_BITS)


@pytest.mark.parametrize("name", ["moe_ds", "moe_ds_skewed"])
def test_full_size_sampled_slots(name):
    import torch
    w = MOE_WORKLOADS[name]
    c = Case(w)
    print("moe full size %s N=%d" % (name, c.N), flush=True)
    out = c.fused(ua.MOE_INTERLEAVED, 4)
    # layout on the device: served rows written, the rest still the sentinel
    rows = out.view(torch.int16).view(w.P * w.T * w.k, w.hidden)
    served = torch.zeros(w.P * w.T * w.k, dtype=torch.bool, device="cuda")
    served[c.drs.long()] = True
    sent = rows == MOE_SENTINEL_BITS
    assert bool(sent[~served].all()) and not bool(sent[served].any())
    # values: 96 seeded served slots over the experts, against the oracle
    rng = np.random.default_rng(w.seed + 1000)
    pick = np.sort(rng.choice(c.N, size=96, replace=False))
    ref_slots = mo.rank_slots(c.idx, w.rank, w.P, w.E)[pick]
    vals = mo.slot_values(c.x, c.idx, c.tw, c.W1, c.W2, w.rank, w.P, w.E, ref_slots)
    got = _f64(_host_bits(rows[c.drs.long()[torch.from_numpy(pick).cuda()]].view(torch.bfloat16)))
    _assert_close(got.reshape(len(pick), w.hidden), vals, name)
    # the other schedule, bit-identical
    out2 = c.fused(ua.MOE_EXPERT_WAVE, 4)
    assert bool(torch.equal(out2.view(torch.int16), out.view(torch.int16)))
