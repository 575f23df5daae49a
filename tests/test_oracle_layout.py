"""Pins of the oracle's post-attention All-to-All placement (CPU only).

Fig. 5 of the review page of the X-Stage paper (steps d-e): after attention the
All-to-All restores the sequence partition, so destination rank p receives, for
every head, the rows of its own sequence chunk.  Reading: rank r owns global
heads [r*Hl, (r+1)*Hl), rank p owns rows [p*S/P, (p+1)*S/P), and the
destination buffer is [B][P][S/P][H][d].
"""
import numpy as np
import pytest

import oracle
from ua_inputs import WORKLOADS, make_qkv


def _all_rows(B, S, Hl):
    bb, hh, ss = np.meshgrid(np.arange(B), np.arange(Hl), np.arange(S), indexing="ij")
    return np.stack([bb.ravel(), hh.ravel(), ss.ravel()], axis=1)


def test_hand_worked_small_case():
    # B=1, S=4, H=4, P=2, d=1: dest is [1][2][2][4][1]; offset = (p*2 + i)*4 + g.
    # Rank 0 owns heads 0,1; rank 1 owns heads 2,3.  Rows 0,1 go to p=0, rows
    # 2,3 to p=1 (i = s - 2).  Worked by hand from the definition above.
    cases = {  # (rank, s, h_l) -> offset
        (0, 0, 0): 0, (0, 0, 1): 1, (0, 1, 0): 4, (0, 1, 1): 5,
        (0, 2, 0): 8, (0, 2, 1): 9, (0, 3, 0): 12, (0, 3, 1): 13,
        (1, 0, 0): 2, (1, 0, 1): 3, (1, 1, 0): 6, (1, 1, 1): 7,
        (1, 2, 0): 10, (1, 2, 1): 11, (1, 3, 0): 14, (1, 3, 1): 15,
    }
    for (r, s, h), off in cases.items():
        assert oracle.dest_offset(0, s, h, 1, 4, 4, 1, 2, r) == off


@pytest.mark.parametrize("name", ["tiny", "dit_image"])
def test_rank_map_is_a_bijection_onto_its_head_slots(name):
    w = WORKLOADS[name]
    rows = _all_rows(w.B, w.S, w.Hl)
    offs = oracle.dest_offsets(rows, w.B, w.S, w.H, w.d, w.P, w.rank)
    assert np.all(offs >= 0)
    assert np.all(offs % w.d == 0)
    slots = offs // w.d                        # row slots of the [B][P][S/P][H] grid
    assert len(np.unique(slots)) == len(slots)  # injective
    g = slots % w.H
    assert np.all((g >= w.rank * w.Hl) & (g < (w.rank + 1) * w.Hl))  # only own heads
    assert len(slots) == w.B * w.S * w.Hl       # covers every owned slot
    # Closed-form inverse: slot -> (b, p, i, g) -> s = p*S/P + i, h_l = g - r*Hl.
    chunk = w.S // w.P
    i = (slots // w.H) % chunk
    p = (slots // (w.H * chunk)) % w.P
    b = slots // (w.H * chunk * w.P)
    np.testing.assert_array_equal(b, rows[:, 0])
    np.testing.assert_array_equal(g - w.rank * w.Hl, rows[:, 1])
    np.testing.assert_array_equal(p * chunk + i, rows[:, 2])


def test_all_ranks_tile_the_buffer_as_bshd():
    # Over all ranks the destination is exactly a [B][S][H][d] tensor:
    # offset == ((b*S + s)*H + g)*d, and every slot is hit once.
    B, S, H, d, P = 2, 24, 6, 4, 3
    Hl = H // P
    rows = _all_rows(B, S, Hl)
    seen = []
    for r in range(P):
        offs = oracle.dest_offsets(rows, B, S, H, d, P, r)
        want = ((rows[:, 0] * S + rows[:, 2]) * H + r * Hl + rows[:, 1]) * d
        np.testing.assert_array_equal(offs, want)
        seen.append(offs)
    seen = np.concatenate(seen)
    assert len(np.unique(seen)) == B * S * H


def test_single_rank_is_identity():
    B, S, H, d = 2, 10, 3, 8
    rows = _all_rows(B, S, H)
    offs = oracle.dest_offsets(rows, B, S, H, d, 1, 0)
    np.testing.assert_array_equal(offs, ((rows[:, 0] * S + rows[:, 2]) * H + rows[:, 1]) * d)


def test_invalid_arguments_are_rejected():
    assert oracle.dest_offset(0, 0, 0, 1, 6, 4, 8, 4, 0) == -1  # S % P != 0
    assert oracle.dest_offset(0, 0, 0, 1, 8, 6, 8, 4, 0) == -1  # H % P != 0
    assert oracle.dest_offset(0, 0, 0, 1, 8, 4, 8, 2, 2) == -1  # rank >= P
    assert oracle.dest_offset(0, 8, 0, 1, 8, 4, 8, 2, 0) == -1  # s >= S
    assert oracle.dest_offset(0, 0, 2, 1, 8, 4, 8, 2, 0) == -1  # h_l >= Hl
    assert oracle.dest_offset(1, 0, 0, 1, 8, 4, 8, 2, 0) == -1  # b >= B


def test_permute_copies_bits_and_leaves_other_slots():
    B, S, H, d, P, r = 2, 16, 8, 8, 4, 2
    Hl = H // P
    O, _, _ = make_qkv(B, S, Hl, d, 40)
    dest = np.full(B * S * H * d, 0x7FD5, np.uint16)
    oracle.permute(O, H, P, r, dest)
    view = dest.reshape(B, S, H, d)     # the BSHD identity of the layout
    np.testing.assert_array_equal(view[:, :, r * Hl:(r + 1) * Hl], O)
    others = np.delete(view, np.s_[r * Hl:(r + 1) * Hl], axis=2)
    assert np.all(others == 0x7FD5)


# ---- the pre-attention exchange (Fig. 5 steps a-c): source rank p holds rows
# [p*S/P, (p+1)*S/P) of all H heads, laid out [B][P][S/P][H][d]; rank r takes
# its heads [r*Hl, (r+1)*Hl) of every row.

def test_gather_hand_worked_small_case():
    # B=1, S=4, H=4, P=2, d=1, X[j] = j: X is [1][2][2][4][1], element
    # (p, i, g) at (p*2 + i)*4 + g.  Rank 1 owns heads 2, 3; its row s comes
    # from region p = s // 2, local row i = s % 2.  Worked by hand.
    X = np.arange(16, dtype=np.uint16).reshape(1, 2, 2, 4, 1)
    want = {0: [[0, 1], [4, 5], [8, 9], [12, 13]],
            1: [[2, 3], [6, 7], [10, 11], [14, 15]]}
    for r in (0, 1):
        got = oracle.gather(X, 4, 2, r)
        assert got.shape == (1, 4, 2, 1)
        np.testing.assert_array_equal(got[0, :, :, 0], np.array(want[r], dtype=np.uint16))


def test_gather_over_all_ranks_reassembles_the_input():
    # concatenating every rank's heads restores X read as [B][S][H][d]
    B, S, H, d, P = 2, 24, 6, 4, 3
    X, _, _ = make_qkv(B, S, H, d, 41)
    parts = [oracle.gather(X.reshape(B, P, S // P, H, d), H, P, r) for r in range(P)]
    np.testing.assert_array_equal(np.concatenate(parts, axis=2), X)


def test_gather_is_the_inverse_of_permute():
    # gather then permute writes back exactly the rank's slots of X
    B, S, H, d, P, r = 2, 16, 8, 8, 4, 3
    X, _, _ = make_qkv(B, S, H, d, 42)
    loc = oracle.gather(X, H, P, r)
    dest = np.full(B * S * H * d, 0x7FD5, np.uint16)
    oracle.permute(loc, H, P, r, dest)
    view = dest.reshape(B, S, H, d)
    Hl = H // P
    np.testing.assert_array_equal(view[:, :, r * Hl:(r + 1) * Hl], X[:, :, r * Hl:(r + 1) * Hl])
    assert np.all(np.delete(view, np.s_[r * Hl:(r + 1) * Hl], axis=2) == 0x7FD5)


def test_gather_rejects_bad_arguments():
    X = np.zeros((1, 8, 4, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle.gather(X, 4, 3, 0)        # H % P
    with pytest.raises(ValueError):
        oracle.gather(X, 4, 2, 2)        # rank >= P
    with pytest.raises(ValueError):
        oracle.gather(X, 6, 2, 0)        # H does not match X
