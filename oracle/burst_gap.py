"""Burst-Gap relations of the X-Stage paper (arXiv 2607.23264), as plain formulas.

TEST / MEASUREMENT INFRASTRUCTURE ONLY.  Context for the fused epilogue: an
output-tile owner issues a burst of stores of volume V, then its next Q-loop
is a gap G during which accepted stores keep draining.  The relations below are
the ones the pith.science review page states in its core-claim section and
parameter ledger; the printed values they are pinned against live in
``tests/golden/xstage_ledger.txt``.

Units are SI throughout: bytes, seconds, bytes/second.
"""
from __future__ import annotations


def issue_time(V: float, G: float, R: float, T0: float) -> float:
    """Sender-visible issue time of a burst V after a producer gap G (Eq. 3):
    the larger of the backpressure-free floor T0 and the part of the drain V/R
    that the gap did not already cover."""
    return max(T0, V / R - G)


def recovery_gap(V: float, R: float, T0: float) -> float:
    """Smallest gap that brings the next burst back to the floor T0: [V/R - T0]+."""
    return max(0.0, V / R - T0)


def single_burst_backlog(V: float, R: float, T0: float) -> float:
    """Bytes still queued when a burst finishes issuing at the floor: [V - R*T0]+.
    The capacity bound of Eq. 10 asks this to stay within the outstanding
    capacity Q."""
    return max(0.0, V - R * T0)


def rate_bound_ok(V: float, G: float, R: float, T0: float) -> bool:
    """Rate bound of Eq. 10: periodic bursts of V every T0 + G sustain <= R."""
    return V / (T0 + G) <= R


def convergence_seq_len(V: float, R: float, T0: float, sigma: float, kv_tile: int) -> float:
    """Sequence length at which one Q-loop (sigma seconds per KV tile of
    ``kv_tile`` keys) already spans the recovery gap: G*/sigma * kv_tile.
    This is the reading used for the bound M*_ub of Eq. 20 / Fig. 11."""
    return recovery_gap(V, R, T0) / sigma * kv_tile
