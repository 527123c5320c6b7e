"""Pins of the MQA logits oracle (oracle/mqa.py) against things other than itself:
the pinned GEMM oracle, exact rationals, closed forms and invariants.  Each
catches a plausible slip: a dropped or extra head, the max applied after the
weights, a transposed head/key role, a wrong scale block or nibble, a window off
by one, the wrong key group."""
from fractions import Fraction

import numpy as np
import pytest

import exact
import oracle
from oracle import mqa

D = 128


def _rng(seed):
    return np.random.default_rng(seed)


def _e4m3_codes(r, rows):
    c = r.integers(0, 256, (rows, D), dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38          # no NaN codes
    return c


def _operands(fmt, r, T, H, rows_k):
    if fmt == "e4m3":
        Q, K = _e4m3_codes(r, T * H), _e4m3_codes(r, rows_k)
        sq = r.integers(118, 136, (T * H, 1), dtype=np.uint8)
        sk = r.integers(118, 136, (rows_k, 1), dtype=np.uint8)
    else:
        Q = r.integers(0, 256, (T * H, D // 2), dtype=np.uint8)
        K = r.integers(0, 256, (rows_k, D // 2), dtype=np.uint8)
        sq = r.integers(118, 136, (T * H, D // 32), dtype=np.uint8)
        sk = r.integers(118, 136, (rows_k, D // 32), dtype=np.uint8)
    return Q, sq, K, sk


def _deq(fmt, codes, sf):
    if fmt == "e4m3":
        return exact.dequant_e4m3(codes, sf, 1, 128)
    return exact.dequant_e2m1(codes, sf, D)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_one_head_unit_weight_is_the_relu_of_the_gemm(fmt):
    """H = 1, w = 1: L = max(0, Q K^T), Q K^T from the pinned GEMM oracle (FP4
    directly; FP8 with per-row key scales through the FP4-independent exact path)."""
    r = _rng(1)
    T, S = 6, 40
    Q, sq, K, sk = _operands(fmt, r, T, 1, S)
    W = np.ones((T, 1), dtype=np.float32)
    L = mqa.mqa_logits(fmt, Q, oracle.pack_scales(sq), K, oracle.pack_scales(sk), W,
                       np.zeros(T), np.full(T, S), S, 1, T, S)
    if fmt == "e2m1":
        G = oracle.gemm_fp4(Q, oracle.pack_scales(sq), K, oracle.pack_scales(sk), D)
    else:
        G = _deq(fmt, Q, sq) @ _deq(fmt, K, sk).T
    assert np.allclose(L, np.maximum(G, 0.0), rtol=1e-14, atol=0)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_exact_rational_brute_force(fmt):
    """Tiny case summed in exact rationals: element values from library
    conversions (tests/exact.py), weights dyadic so every step is exact."""
    r = _rng(2)
    T, H, S = 3, 4, 7
    Q, sq, K, sk = _operands(fmt, r, T, H, S)
    W = (r.integers(-8, 9, (T, H)) / 4.0).astype(np.float32)
    ks = np.array([0, 2, 3])
    ke = np.array([7, 5, 3])
    L = mqa.mqa_logits(fmt, Q, oracle.pack_scales(sq), K, oracle.pack_scales(sk), W, ks, ke,
                       S, H, T, S)
    q, k = _deq(fmt, Q, sq), _deq(fmt, K, sk)
    for t in range(T):
        for s in range(S):
            if not (ks[t] <= s < ke[t]):
                assert L[t, s] == -np.inf
                continue
            tot = Fraction(0)
            for h in range(H):
                dot = sum((Fraction(float(a)) * Fraction(float(b))
                           for a, b in zip(q[t * H + h], k[s])), Fraction(0))
                tot += Fraction(float(W[t, h])) * max(dot, Fraction(0))
            assert abs(Fraction(L[t, s]) - tot) <= abs(tot) * Fraction(1, 2 ** 50)


def test_nonnegative_operands_contract_heads_first():
    """With every code non-negative the max never acts, so L = (sum_h w_h q_h) . k:
    the heads contracted before the keys, a different order of the same sums."""
    r = _rng(3)
    T, H, S = 4, 8, 50
    Q, sq, K, sk = _operands("e4m3", r, T, H, S)
    Q &= 0x7F
    K &= 0x7F
    W = r.standard_normal((T, H)).astype(np.float32)
    L = mqa.mqa_logits("e4m3", Q, oracle.pack_scales(sq), K, oracle.pack_scales(sk), W,
                       np.zeros(T), np.full(T, S), S, H, T, S)
    q, k = _deq("e4m3", Q, sq), _deq("e4m3", K, sk)
    for t in range(T):
        qw = W[t].astype(np.float64) @ q[t * H:(t + 1) * H]
        assert np.allclose(L[t], k @ qw, rtol=1e-12, atol=0)


def test_scale_only_closed_form_fp4():
    """Unit codes (e2m1 1.0) with one scale byte per 32-block: q_h . k_s =
    32 * sum_b 2^(eq(h, b) + ek(s, b)), so L = sum_h w_h * that; pins the scale
    block of every 32 elements and the nibble pairing."""
    r = _rng(4)
    T, H, S = 2, 3, 5
    Q = np.full((T * H, D // 2), 0x22, dtype=np.uint8)
    K = np.full((S, D // 2), 0x22, dtype=np.uint8)
    eq = r.integers(-4, 5, (T * H, 4))
    ek = r.integers(-4, 5, (S, 4))
    W = np.array([[1.0, -2.0, 0.5], [3.0, 0.25, -1.0]], dtype=np.float32)
    L = mqa.mqa_logits("e2m1", Q, oracle.pack_scales((eq + 127).astype(np.uint8)), K,
                       oracle.pack_scales((ek + 127).astype(np.uint8)), W, np.zeros(T),
                       np.full(T, S), S, H, T, S)
    for t in range(T):
        for s in range(S):
            want = sum(float(W[t, h]) * 32.0 * np.sum(2.0 ** (eq[t * H + h] + ek[s]))
                       for h in range(H))
            assert L[t, s] == want


def test_negative_scores_are_cut_before_the_weights():
    """A head whose dot product is negative contributes nothing, whatever the sign
    of its weight; the max acts per head, not on the weighted sum."""
    T, H, S = 1, 2, 1
    Q = np.zeros((2, D), dtype=np.uint8)
    Q[0, :] = 0x38                     # +1
    Q[1, :] = 0xB8                     # -1
    K = np.full((1, D), 0x38, dtype=np.uint8)
    one = oracle.pack_scales(np.full((2, 1), 127, dtype=np.uint8))
    for w in ([1.0, 1.0], [1.0, -1.0], [-1.0, 5.0]):
        L = mqa.mqa_logits("e4m3", Q, one, K, one[:, :1], np.array([w], dtype=np.float32),
                           [0], [1], S, H, 1, S)
        assert L[0, 0] == w[0] * 128.0


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_head_permutation_and_weight_linearity(fmt):
    r = _rng(5)
    T, H, S = 3, 8, 30
    Q, sq, K, sk = _operands(fmt, r, T, H, S)
    W1 = (r.integers(-64, 65, (T, H)) / 16.0).astype(np.float32)   # dyadic: W1 + W2 is exact
    W2 = (r.integers(-64, 65, (T, H)) / 16.0).astype(np.float32)
    args = (K, oracle.pack_scales(sk))
    full = (np.zeros(T), np.full(T, S), S, H, T, S)
    L1 = mqa.mqa_logits(fmt, Q, oracle.pack_scales(sq), *args, W1, *full)
    L2 = mqa.mqa_logits(fmt, Q, oracle.pack_scales(sq), *args, W2, *full)
    L12 = mqa.mqa_logits(fmt, Q, oracle.pack_scales(sq), *args,
                         (W1.astype(np.float64) + W2).astype(np.float32), *full)
    assert np.allclose(L12, L1 + L2, rtol=0, atol=1e-13 * (np.abs(L1).max() + np.abs(L2).max()))
    p = r.permutation(H)
    rows = (np.arange(T)[:, None] * H + p[None, :]).ravel()
    Lp = mqa.mqa_logits(fmt, Q[rows], oracle.pack_scales(sq[rows]), *args, W1[:, p], *full)
    assert np.allclose(Lp, L1, rtol=1e-13, atol=0)


def test_windows_and_key_groups():
    """Outside [ks, ke) every entry is -inf (an empty window gives a row of -inf);
    query t reads key group t // q_per_group, which equals a call on that group's
    keys alone."""
    r = _rng(6)
    T, H, S, per = 6, 4, 20, 2
    groups = T // per
    Q, sq, K, sk = _operands("e4m3", r, T, H, groups * S)
    W = r.standard_normal((T, H)).astype(np.float32)
    ks = np.array([0, 3, 5, 5, 0, 19])
    ke = np.array([20, 4, 5, 12, 1, 20])
    L = mqa.mqa_logits("e4m3", Q, oracle.pack_scales(sq), K, oracle.pack_scales(sk), W, ks, ke,
                       S, H, per, S)
    for t in range(T):
        inside = (np.arange(S) >= ks[t]) & (np.arange(S) < ke[t])
        assert np.all(L[t, ~inside] == -np.inf) and np.all(np.isfinite(L[t, inside]))
    for g in range(groups):
        qs = slice(g * per, (g + 1) * per)
        qrows = slice(g * per * H, (g + 1) * per * H)
        Lg = mqa.mqa_logits("e4m3", Q[qrows], oracle.pack_scales(sq[qrows]), K[g * S:(g + 1) * S],
                            oracle.pack_scales(sk[g * S:(g + 1) * S]), W[qs], ks[qs], ke[qs],
                            S, H, per, S)
        assert np.array_equal(Lg, L[qs])


def test_denominator_bounds_every_logit():
    r = _rng(7)
    T, H, S = 3, 8, 25
    Q, sq, K, sk = _operands("e2m1", r, T, H, S)
    W = r.standard_normal((T, H)).astype(np.float32)
    L = mqa.mqa_logits("e2m1", Q, oracle.pack_scales(sq), K, oracle.pack_scales(sk), W,
                       np.zeros(T), np.full(T, S), S, H, T, S)
    den = mqa.norm_denominator("e2m1", Q, oracle.pack_scales(sq), K, oracle.pack_scales(sk), W,
                               S, H, T, S)
    assert np.all(np.abs(L) <= den * (1 + 1e-12)) and np.all(den > 0)
