"""fp64 CPU oracle of one expert-parallel rank's MoE expert path with the
Combine exchange: the computation the pages' MegaMoE kernel fuses.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and by the benchmark's
CPU-baseline leg, never by the product package.  It shares no code with the
HIP path; both sides only share the seeded input generator (moe_inputs.py).

What it follows (X-Stage paper, arXiv 2607.23264; the arXiv abstract page,
Abstract, and the pith.science review page, "If this is right" and Figs. 4,
8, 9): each rank runs its local experts' two linear layers on the tokens
routed to them, Linear-1 and Linear-2, and the Combine sends every expert
output back to the rank that owns its token.  The pages fix neither the
activation nor the layouts; the plainest readings, also stated in the design
notes, are:
  * an expert is the gated feed-forward block of the DeepSeek-style models
    the pages' MegaMoE serves: h = x W1^T with W1 [2*inter][hidden] (rows
    0..inter-1 the gate, the rest the up projection), a = SiLU(gate) * up,
    y = a W2^T with W2 [hidden][inter]; SiLU(z) = z / (1 + exp(-z));
  * rank r holds experts r*E_l .. r*E_l+E_l-1 (E_l = E/P), a contiguous block;
  * token t of source rank p chose experts topk_idx[p][t][0..k-1] with
    weights topk_w[p][t][0..k-1]; the Combine stores topk_w[p][t][j] * y into
    slot (t, j) of region p of the combine buffer [P][T][k][hidden], one slot
    per choice, and the source rank sums a token's k slots afterwards (that
    sum is outside the fused path);
  * everything here is fp64 on the exactly widened bf16 inputs, with no
    intermediate rounding (the plain definition).
"""
from __future__ import annotations

import numpy as np


def widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def silu(z):
    """SiLU (swish): z * sigmoid(z) = z / (1 + exp(-z))."""
    return z / (1.0 + np.exp(-z))


def expert_ffn(x_rows: np.ndarray, W1: np.ndarray, W2: np.ndarray) -> np.ndarray:
    """One expert on a block of token rows (all float64): Linear-1, the gated
    activation, Linear-2.  x_rows [n][hidden], W1 [2*inter][hidden],
    W2 [hidden][inter] -> [n][hidden]."""
    inter = W1.shape[0] // 2
    h = x_rows @ W1.T                    # Linear-1: [n][2*inter]
    a = silu(h[:, :inter]) * h[:, inter:]
    return a @ W2.T                      # Linear-2: [n][hidden]


def rank_slots(topk_idx: np.ndarray, rank: int, P: int, E: int) -> np.ndarray:
    """The combine slots this rank's experts serve, as int64 rows
    (local expert e, source rank p, token t, choice j), ordered by e, then p,
    t, j.  topk_idx is [P][T][k] (global expert ids)."""
    E_l = E // P
    out = []
    for e in range(E_l):
        p, t, j = np.nonzero(topk_idx == rank * E_l + e)
        for s in sorted(zip(p.tolist(), t.tolist(), j.tolist())):
            out.append((e,) + s)
    return np.asarray(out, dtype=np.int64).reshape(-1, 4)


def slot_values(x_bits, topk_idx, topk_w, W1_bits, W2_bits, rank, P, E, slots=None) -> np.ndarray:
    """fp64 combine values of this rank's slots: topk_w[p,t,j] * FFN_e(x[p,t])
    for every row (e, p, t, j) of `slots` (default: all of rank_slots)."""
    if slots is None:
        slots = rank_slots(topk_idx, rank, P, E)
    hidden = x_bits.shape[-1]
    out = np.empty((len(slots), hidden))
    for e in np.unique(slots[:, 0]) if len(slots) else []:
        sel = np.nonzero(slots[:, 0] == e)[0]
        _, p, t, j = slots[sel].T
        y = expert_ffn(widen(x_bits[p, t]), widen(W1_bits[e]), widen(W2_bits[e]))
        out[sel] = topk_w[p, t, j].astype(np.float64)[:, None] * y
    return out


def combine_buffer(x_bits, topk_idx, topk_w, W1_bits, W2_bits, rank, P, E) -> np.ndarray:
    """The combine buffer [P][T][k][hidden] after this rank's expert path: its
    slots hold their fp64 values, every other slot NaN (untouched)."""
    Pp, T, k = topk_idx.shape
    out = np.full((Pp, T, k, x_bits.shape[-1]), np.nan)
    slots = rank_slots(topk_idx, rank, P, E)
    vals = slot_values(x_bits, topk_idx, topk_w, W1_bits, W2_bits, rank, P, E, slots)
    out[slots[:, 1], slots[:, 2], slots[:, 3]] = vals
    return out


def slot_offsets(slots: np.ndarray, T: int, k: int, hidden: int) -> np.ndarray:
    """Element offset of each slot's row in the combine buffer [P][T][k][hidden]."""
    return ((slots[:, 1] * T + slots[:, 2]) * k + slots[:, 3]) * hidden
