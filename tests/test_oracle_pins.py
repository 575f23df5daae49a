"""Pins of the fp64 oracle against things other than itself (CPU only).

The pages print no numeric attention example, so the oracle's arithmetic is
pinned by: a 50-digit mpmath brute force without max subtraction on tiny
inputs, closed forms (S=1, S=2, Q=0, uniform V, a dominant key), invariants
(weights sum to 1, joint K/V row permutation, a shared key shift, linearity in
V), and the layout identities of the post-attention All-to-All (Fig. 5 of the
review page of the X-Stage paper, steps d-e).  Each check is chosen so a
plausible slip -- a dropped scale, a wrong sign, an index swap between the
sequence and head axes, a transposed operand, a missing normalisation, an
off-by-one in the rank/row split -- fails at least one of them.
"""
import math

import mpmath
import numpy as np
import pytest

import oracle
from ua_inputs import bf16_bits_to_f32, make_qkv, to_bf16_bits


def _bits(x):
    return to_bf16_bits(np.asarray(x, dtype=np.float32))


def _brute(Qf, Kf, Vf, scale, b, h, s):
    """Softmax attention for one row at 50 digits, no max subtraction."""
    with mpmath.workdps(50):
        S, d = Kf.shape[1], Kf.shape[3]
        sc = mpmath.mpf(scale)
        e = []
        for j in range(S):
            acc = mpmath.mpf(0)
            for k in range(d):
                acc += mpmath.mpf(float(Qf[b, s, h, k])) * mpmath.mpf(float(Kf[b, j, h, k]))
            e.append(mpmath.exp(acc * sc))
        tot = mpmath.fsum(e)
        return [float(mpmath.fsum(e[j] * mpmath.mpf(float(Vf[b, j, h, k])) for j in range(S)) / tot)
                for k in range(d)]


@pytest.mark.parametrize("B,S,Hl,d,seed", [(1, 1, 1, 4, 10), (2, 5, 3, 3, 11),
                                           (1, 17, 2, 16, 12), (2, 64, 2, 8, 13)])
def test_matches_mpmath_brute_force(B, S, Hl, d, seed):
    Q, K, V = make_qkv(B, S, Hl, d, seed)
    scale = 1.0 / math.sqrt(d)
    got = oracle.attn_all(Q, K, V, scale)
    Qf, Kf, Vf = (bf16_bits_to_f32(t) for t in (Q, K, V))
    for b in range(B):
        for h in range(Hl):
            for s in range(S):
                ref = np.array(_brute(Qf, Kf, Vf, scale, b, h, s))
                np.testing.assert_allclose(got[b, s, h], ref, rtol=1e-13, atol=1e-14)


def test_brute_force_with_non_default_scale_and_large_values():
    # Logits of order 10: exercises the exponent range without max subtraction.
    rng = np.random.default_rng(5)
    B, S, Hl, d = 1, 9, 2, 4
    Q = _bits(rng.standard_normal((B, S, Hl, d)) * 3)
    K = _bits(rng.standard_normal((B, S, Hl, d)) * 3)
    V = _bits(rng.standard_normal((B, S, Hl, d)))
    got = oracle.attn_all(Q, K, V, 0.7)
    Qf, Kf, Vf = (bf16_bits_to_f32(t) for t in (Q, K, V))
    for h in range(Hl):
        for s in range(S):
            np.testing.assert_allclose(got[0, s, h], _brute(Qf, Kf, Vf, 0.7, 0, h, s),
                                       rtol=1e-13, atol=1e-14)


def test_weights_are_a_distribution():
    Q, K, V = make_qkv(2, 300, 3, 64, 21)
    for (b, h, s) in [(0, 0, 0), (1, 2, 299), (0, 1, 150), (1, 0, 7)]:
        w = oracle.softmax_row(Q, K, 0.125, b, h, s)
        assert np.all(w >= 0.0)
        assert abs(w.sum() - 1.0) < 1e-12


def test_single_key_returns_its_value_row():
    Q, K, V = make_qkv(2, 1, 3, 64, 22)
    got = oracle.attn_all(Q, K, V, 0.125)
    np.testing.assert_array_equal(got, oracle.widen(V))


def test_two_keys_closed_form():
    # S = 2: o = v0 + (v1 - v0) * sigmoid(scale * q . (k1 - k0)).
    Q, K, V = make_qkv(1, 2, 2, 32, 23)
    scale = 1.0 / math.sqrt(32)
    got = oracle.attn_all(Q, K, V, scale)
    q, k, v = oracle.widen(Q), oracle.widen(K), oracle.widen(V)
    for h in range(2):
        for s in range(2):
            t = scale * float(np.dot(q[0, s, h], k[0, 1, h] - k[0, 0, h]))
            sig = 1.0 / (1.0 + math.exp(-t))
            want = v[0, 0, h] + (v[0, 1, h] - v[0, 0, h]) * sig
            np.testing.assert_allclose(got[0, s, h], want, rtol=1e-13, atol=1e-15)


def test_zero_query_gives_column_mean_of_v():
    B, S, Hl, d = 1, 257, 2, 64
    _, K, V = make_qkv(B, S, Hl, d, 24)
    Q = np.zeros_like(K)
    got = oracle.attn_all(Q, K, V, 0.125)
    mean = oracle.widen(V).mean(axis=1)  # [B][Hl][d]
    for s in range(S):
        np.testing.assert_allclose(got[:, s], mean, rtol=1e-12, atol=1e-14)


def test_uniform_v_gives_constant_output():
    B, S, Hl, d = 2, 130, 2, 64
    Q, K, _ = make_qkv(B, S, Hl, d, 25)
    c = _bits(np.random.default_rng(26).standard_normal((B, 1, Hl, d)))
    V = np.ascontiguousarray(np.broadcast_to(c, (B, S, Hl, d)))
    got = oracle.attn_all(Q, K, V, 0.125)
    np.testing.assert_allclose(got, np.broadcast_to(oracle.widen(c), got.shape),
                               rtol=1e-12, atol=0)


def test_dominant_key_selects_its_value_and_stays_finite():
    # One key aligned with the query, huge logit (~1e4): the max subtraction
    # must keep exp() finite and the output must be that key's value row.
    B, S, Hl, d = 1, 40, 1, 16
    rng = np.random.default_rng(27)
    Kf = np.zeros((B, S, Hl, d), np.float32)
    Kf[0, :, 0, :] = rng.standard_normal((S, d)) * 0.01
    Kf[0, 13, 0, :] = 0.0
    Kf[0, 13, 0, 3] = 100.0
    Qf = np.zeros((B, S, Hl, d), np.float32)
    Qf[0, :, 0, 3] = 100.0
    Q, K = _bits(Qf), _bits(Kf)
    V = _bits(rng.standard_normal((B, S, Hl, d)))
    got = oracle.attn_all(Q, K, V, 1.0)
    assert np.all(np.isfinite(got))
    for s in range(S):
        np.testing.assert_allclose(got[0, s, 0], oracle.widen(V)[0, 13, 0], rtol=0, atol=1e-12)


def test_joint_key_value_permutation_invariance():
    B, S, Hl, d = 2, 96, 2, 32
    Q, K, V = make_qkv(B, S, Hl, d, 28)
    perm = np.random.default_rng(29).permutation(S)
    a = oracle.attn_all(Q, K, V, 0.2)
    b = oracle.attn_all(Q, np.ascontiguousarray(K[:, perm]), np.ascontiguousarray(V[:, perm]), 0.2)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)


def test_shared_key_shift_invariance():
    # K_j + u for every key adds scale*q.u to every logit of a row: no change.
    # Small integers keep both K and K+u exact in bf16.
    rng = np.random.default_rng(30)
    B, S, Hl, d = 1, 50, 2, 8
    Kf = rng.integers(-4, 5, size=(B, S, Hl, d)).astype(np.float32)
    u = rng.integers(-3, 4, size=(1, 1, Hl, d)).astype(np.float32)
    Qf = rng.integers(-2, 3, size=(B, S, Hl, d)).astype(np.float32) * 0.25
    V = _bits(rng.standard_normal((B, S, Hl, d)))
    a = oracle.attn_all(_bits(Qf), _bits(Kf), V, 0.3)
    b = oracle.attn_all(_bits(Qf), _bits(Kf + u), V, 0.3)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-14)


def test_linear_in_v():
    # Small integers so that V1 + V2 is exact in bf16.
    rng = np.random.default_rng(31)
    B, S, Hl, d = 1, 70, 2, 16
    Q, K, _ = make_qkv(B, S, Hl, d, 32)
    V1 = rng.integers(-8, 9, size=(B, S, Hl, d)).astype(np.float32)
    V2 = rng.integers(-8, 9, size=(B, S, Hl, d)).astype(np.float32)
    o1 = oracle.attn_all(Q, K, _bits(V1), 0.25)
    o2 = oracle.attn_all(Q, K, _bits(V2), 0.25)
    o12 = oracle.attn_all(Q, K, _bits(V1 + V2), 0.25)
    np.testing.assert_allclose(o12, o1 + o2, rtol=1e-12, atol=1e-12)


def test_rows_api_matches_full_and_rejects_bad_rows():
    Q, K, V = make_qkv(2, 33, 3, 16, 33)
    full = oracle.attn_all(Q, K, V, 0.25)
    rows = np.array([[1, 2, 32], [0, 0, 0], [1, 1, 17]])
    got = oracle.attn_rows(Q, K, V, 0.25, rows)
    for n, (b, h, s) in enumerate(rows):
        np.testing.assert_array_equal(got[n], full[b, s, h])
    with pytest.raises(ValueError):
        oracle.attn_rows(Q, K, V, 0.25, np.array([[0, 3, 0]]))
    with pytest.raises(ValueError):
        oracle.attn_rows(Q, K, V, 0.25, np.array([[0, 0, 33]]))


def test_widen_is_exact():
    bits = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F], np.uint16)
    want = [0.0, -0.0, 1.0, -1.0, 3.140625, 2.0 ** -133, 3.3895313892515355e38]
    np.testing.assert_array_equal(oracle.widen(bits), np.array(want))
