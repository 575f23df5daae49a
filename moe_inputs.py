"""Seeded synthetic inputs for the MoE expert path, shared by the tests and the
benchmark.

This module holds no arithmetic of the method: it draws random numbers,
rounds them to bf16 bit patterns and names the workloads.  Both the HIP path
and the CPU oracle receive the arrays it returns; neither imports the other.

Recipe (the pages name no model shapes, give no routing traces and use no
dataset; these tensors stand in for one expert-parallel rank's share of a
DeepSeek-style MoE layer, the kind of model the pages' MegaMoE kernel serves):
  * ``numpy.random.default_rng(seed)`` (PCG64) draws, in this order:
      - x: the tokens of all P ranks, float32 standard normals, [P][T][hidden];
      - the routing: for every token, k distinct experts out of E.  "balanced"
        draws them uniformly; "skewed" draws them with probabilities
        proportional to 1 / (rank_of_expert + 1) ** 1.2 over a random
        permutation of the experts (a few hot experts, a long tail);
      - the routing weights: Dirichlet(1, ..., 1) over the k choices of each
        token, float32;
  * expert g's weights (g the global expert id; rank r holds experts
    r*E_l .. r*E_l+E_l-1) come from their own generators,
    ``default_rng([seed, 1, g])`` for W1_g: [2*inter][hidden] (rows
    0..inter-1 gate, inter..2*inter-1 up, the usual [out][in] layout of a
    linear layer), standard normals scaled by 1/sqrt(hidden), and
    ``default_rng([seed, 2, g])`` for W2_g: [hidden][inter], standard normals
    scaled by 1/sqrt(inter) -- only this rank's E_l = E/P experts;
  * x, W1 and W2 are rounded to bf16 (round to nearest, ties to even) by bit
    arithmetic on the float32 pattern; weights stay float32; expert ids int32.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from ua_inputs import to_bf16_bits

# Raw bf16 bits written into every combine slot before a call (a quiet NaN
# with a payload no arithmetic produces).
MOE_SENTINEL_BITS = 0x7FD5


@dataclass(frozen=True)
class MoeWorkload:
    name: str
    P: int          # expert-parallel ranks (regions of the combine buffer)
    rank: int       # the rank whose experts run here
    T: int          # tokens per rank
    hidden: int
    inter: int      # intermediate size of one expert
    E: int          # experts over all ranks
    k: int          # experts per token
    seed: int
    routing: str = "balanced"   # or "skewed"

    @property
    def E_l(self) -> int:
        return self.E // self.P


def moe_tensors(w: MoeWorkload):
    """x [P][T][hidden] bf16 bits, topk_idx [P][T][k] int32, topk_w [P][T][k]
    float32, W1 [E_l][2*inter][hidden] and W2 [E_l][hidden][inter] bf16 bits."""
    x, topk_idx, topk_w = moe_tokens(w)
    W1, W2 = moe_rank_weights(w, w.rank)
    return x, topk_idx, topk_w, W1, W2


def moe_tokens(w: MoeWorkload):
    """x [P][T][hidden] bf16 bits, topk_idx [P][T][k] int32, topk_w [P][T][k] float32."""
    rng = np.random.default_rng(w.seed)
    x = rng.standard_normal((w.P, w.T, w.hidden), dtype=np.float32)
    n_tok = w.P * w.T
    if w.routing == "balanced":
        keys = rng.random((n_tok, w.E))
        idx = np.argsort(keys, axis=1)[:, : w.k]
    elif w.routing == "skewed":
        order = rng.permutation(w.E)
        pop = np.empty(w.E)
        pop[order] = 1.0 / (np.arange(w.E) + 1.0) ** 1.2
        # k distinct draws per token, weighted by popularity (Gumbel top-k)
        g = rng.gumbel(size=(n_tok, w.E)) + np.log(pop)[None, :]
        idx = np.argsort(-g, axis=1)[:, : w.k]
    else:
        raise ValueError(w.routing)
    topk_idx = idx.astype(np.int32).reshape(w.P, w.T, w.k)
    topk_w = rng.dirichlet(np.ones(w.k), size=n_tok).astype(np.float32).reshape(w.P, w.T, w.k)
    return to_bf16_bits(x), topk_idx, topk_w


def moe_rank_weights(w: MoeWorkload, rank: int):
    """W1 [E_l][2*inter][hidden] and W2 [E_l][hidden][inter] of rank `rank`'s experts."""
    ws = [moe_expert_weights(w, rank * w.E_l + e) for e in range(w.E_l)]
    return np.stack([a for a, _ in ws]), np.stack([b for _, b in ws])


def moe_expert_weights(w: MoeWorkload, g: int):
    """W1_g [2*inter][hidden] and W2_g [hidden][inter] of global expert g, bf16 bits."""
    g1 = np.random.default_rng([w.seed, 1, g])
    W1 = g1.standard_normal((2 * w.inter, w.hidden), dtype=np.float32) * np.float32(w.hidden ** -0.5)
    g2 = np.random.default_rng([w.seed, 2, g])
    W2 = g2.standard_normal((w.hidden, w.inter), dtype=np.float32) * np.float32(w.inter ** -0.5)
    return to_bf16_bits(W1), to_bf16_bits(W2)


# Workloads: one rank of an 8- or 4-way expert-parallel group.  The large
# ones follow the shape of a DeepSeek-style layer (hidden 7168, expert
# intermediate 2048, 256 experts, 8 per token); the small ones fit the oracle.
MOE_WORKLOADS = {
    w.name: w
    for w in [
        MoeWorkload("moe_tiny", P=2, rank=1, T=64, hidden=256, inter=128, E=8, k=2, seed=10),
        MoeWorkload("moe_small", P=4, rank=2, T=512, hidden=1024, inter=512, E=32, k=4, seed=11),
        MoeWorkload("moe_small_skewed", P=4, rank=0, T=512, hidden=1024, inter=512, E=32, k=4, seed=12,
                    routing="skewed"),
        MoeWorkload("moe_ds", P=8, rank=3, T=2048, hidden=7168, inter=2048, E=256, k=8, seed=13),
        # the same tokens and weights as moe_ds (same seed), skewed routing
        MoeWorkload("moe_ds_skewed", P=8, rank=3, T=2048, hidden=7168, inter=2048, E=256, k=8, seed=13,
                    routing="skewed"),
    ]
}
