"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method: it only draws random numbers,
rounds them to bf16 bit patterns and names the workloads.  Both the HIP path and
the CPU oracle receive the arrays it returns; neither imports the other.

Recipe (the pages use no dataset and give no model shapes, so these synthetic
tensors stand in for one Ulysses rank's share of a DiT attention layer):
  * ``numpy.random.default_rng(seed)`` (PCG64) draws float32 standard normals
    for Q, then K, then V, each of shape [B][S][Hl][d] in C order;
  * the "peaky" variant then draws one factor per key row (b, j, h) from
    U(0.5, 2) with the same generator and multiplies K by it in float32;
  * every value is rounded to bf16 (round to nearest, ties to even) by bit
    arithmetic on the float32 pattern.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# Raw bf16 bits written into every destination slot before a call: a quiet NaN
# with a payload no arithmetic produces, so an untouched slot is recognisable.
SENTINEL_BITS = 0x7FD5


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S: int
    H: int       # total heads over all ranks
    P: int       # ranks of the Ulysses group (regions of the destination buffer)
    rank: int
    d: int
    seed: int
    peaky_k: bool = False   # K rows scaled by U(0.5, 2)
    sampled: bool = False   # the oracle checks sampled rows instead of all rows

    @property
    def Hl(self) -> int:
        return self.H // self.P

    @property
    def flops(self) -> int:
        """QK^T plus PV, non-causal: 4 * S^2 * d per (batch, local head)."""
        return 4 * self.S * self.S * self.d * self.Hl * self.B

    @property
    def out_bytes(self) -> int:
        """bf16 bytes this rank writes into the destination buffer."""
        return self.B * self.S * self.Hl * self.d * 2

    @property
    def dest_bytes(self) -> int:
        return self.B * self.S * self.H * self.d * 2


# Workloads: one Ulysses rank's attention at DiT-like shapes.  Sizes follow the
# sequence range the paper measures (up to M = 65,536 tokens, Fig. 11).
WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", B=1, S=512, H=4, P=2, rank=0, d=64, seed=0),
        Workload("dit_image", B=1, S=4096, H=24, P=8, rank=3, d=128, seed=1),
        Workload("dit_long", B=1, S=16384, H=24, P=8, rank=5, d=128, seed=2,
                 peaky_k=True, sampled=True),
        Workload("video_dit", B=1, S=65536, H=40, P=8, rank=7, d=128, seed=3,
                 sampled=True),
        Workload("mixed", B=2, S=32768, H=24, P=4, rank=1, d=64, seed=4,
                 sampled=True),
    ]
}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.  Finite input."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact bf16 bits -> float32 values (for building test inputs only)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def make_qkv(B: int, S: int, Hl: int, d: int, seed: int, peaky_k: bool = False):
    """Q, K, V as uint16 bf16 bits, each [B][S][Hl][d] (recipe in the module doc)."""
    rng = np.random.default_rng(seed)
    shape = (B, S, Hl, d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if peaky_k:
        f = rng.uniform(0.5, 2.0, size=(B, S, Hl)).astype(np.float32)
        k = k * f[..., None]
    return to_bf16_bits(q), to_bf16_bits(k), to_bf16_bits(v)


def workload_qkv(w: Workload):
    return make_qkv(w.B, w.S, w.Hl, w.d, w.seed, w.peaky_k)


def sampled_rows(w: Workload, n_per_head: int = 256) -> np.ndarray:
    """Query rows checked against the oracle, as (b, h_l, s) int64 triples.

    Per (b, h_l): ``n_per_head`` distinct rows from default_rng(seed + 1000),
    plus row 0, row S-1 and both rows at every destination-region boundary.
    Without sampling, every row.
    """
    B, S, Hl, P = w.B, w.S, w.Hl, w.P
    if not w.sampled:
        bb, hh, ss = np.meshgrid(np.arange(B), np.arange(Hl), np.arange(S), indexing="ij")
        return np.stack([bb.ravel(), hh.ravel(), ss.ravel()], axis=1).astype(np.int64)
    rng = np.random.default_rng(w.seed + 1000)
    chunk = S // P
    edges = {0, S - 1}
    for p in range(1, P):
        edges.update({p * chunk - 1, p * chunk})
    out = []
    for b in range(B):
        for h in range(Hl):
            pick = set(rng.choice(S, size=min(n_per_head, S), replace=False).tolist())
            for s in sorted(pick | edges):
                out.append((b, h, s))
    return np.asarray(out, dtype=np.int64)
