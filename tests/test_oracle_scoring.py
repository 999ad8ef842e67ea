"""Pins for the oracle's query prep, key projection and scoring.

The projected score of the JSSA article (section "打分误差的定义") is
s_hat = q_bar^T P k with P = M^T M, which equals (M q_bar).(M k); the error against
the full score s = q_bar^T k is q_bar^T (I - P) k. The checks below use bases and
values for which every quantity is exact in binary, so the oracle's results can be
compared with exact rational arithmetic.
"""
from fractions import Fraction

import numpy as np

from oracle import jssa
from oracle.numerics import bf16_to_f32, round_to_bf16


def _bf16(vals):
    return round_to_bf16(np.asarray(vals, dtype=np.float64))


def _exact_round_bf16(fr: Fraction) -> float:
    """Round a rational to 8 significant bits, ties to even, with integer arithmetic."""
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    scaled = a * 128                     # [128, 256)
    fl = scaled.numerator // scaled.denominator
    rem = scaled - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(Fraction(fl) / 128 * Fraction(2) ** e)


H4 = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]], dtype=np.float64) / 2.0


def test_hadamard_basis_identity_exact():
    rng = np.random.default_rng(1)
    M = H4[:2].astype(np.float32)                      # orthonormal rows, exact entries
    P = H4[:2].T @ H4[:2]
    for _ in range(50):
        qh = _bf16(rng.integers(-8, 9, size=(4, 4)))     # G=4 heads, d=4, small integers
        keys = _bf16(rng.integers(-8, 9, size=(16, 4)))
        q_bar = jssa.mean_query(qh)
        q_hat = jssa.project_query(q_bar, M)
        kproj = jssa.project_keys(keys, M)
        s_hat = jssa.score_positions(q_hat, kproj)
        qb = bf16_to_f32(qh).astype(np.float64).mean(axis=0)
        kf = bf16_to_f32(keys).astype(np.float64)
        # s_hat = q_bar^T P k exactly (all values are small dyadic rationals)
        want = kf @ (P @ qb)
        assert np.array_equal(s_hat.astype(np.float64), want)
        # the projection error is q_bar^T (I-P) k
        full = kf @ qb
        assert np.array_equal(full - s_hat, kf @ ((np.eye(4) - P) @ qb))


def test_full_rank_signed_permutation_preserves_scores():
    # With r = d, P = I: the projected score equals the textbook q_bar . k. A
    # non-symmetric signed permutation catches a transposed basis anywhere.
    rng = np.random.default_rng(2)
    d = 128
    perm = rng.permutation(d)
    sign = rng.choice([-1.0, 1.0], size=d)
    M = np.zeros((d, d), dtype=np.float32)
    M[np.arange(d), perm] = sign
    qh = _bf16(rng.standard_normal((4, d)))
    keys = _bf16(rng.standard_normal((300, d)))
    s_hat = jssa.score_positions(jssa.project_query(jssa.mean_query(qh), M), jssa.project_keys(keys, M))
    qb = jssa.mean_query(qh).astype(np.float64)
    want = (bf16_to_f32(keys).astype(np.float64) @ qb).astype(np.float32)
    assert np.max(np.abs(s_hat.astype(np.float64) - want)) <= 2e-6 * np.max(np.abs(want))
    assert np.array_equal(jssa.select_topk(s_hat, 17), jssa.select_topk(want, 17))


def test_identity_basis_scores_are_rounded_exact_dots():
    rng = np.random.default_rng(3)
    d = 128
    qh = _bf16(rng.standard_normal((4, d)))
    keys = _bf16(rng.standard_normal((8, d)))
    M = np.eye(d, dtype=np.float32)
    q_bar = jssa.mean_query(qh)
    kproj = jssa.project_keys(keys, M)
    assert np.array_equal(kproj, keys)          # projecting onto I_d keeps bf16 keys
    s = jssa.score_positions(jssa.project_query(q_bar, M), kproj)
    kf = bf16_to_f32(keys)
    for j in range(8):
        exact = sum(Fraction(float(q_bar[i])) * Fraction(float(kf[j, i])) for i in range(d))
        assert s[j] == np.float32(float(exact))


def test_mean_query_is_fp32_mean():
    qh = _bf16([[1.0, 2.0, -3.0], [3.0, 2.0, 5.0], [0.5, 0.25, 1.0], [0.5, -0.25, 1.0]])
    assert np.array_equal(jssa.mean_query(qh), np.array([1.25, 1.0, 1.0], dtype=np.float32))


def test_project_keys_exact_rational_rounding():
    rng = np.random.default_rng(4)
    d, r = 128, 16
    M = rng.standard_normal((r, d)).astype(np.float32)
    keys = _bf16(rng.standard_normal((3, d)))
    got = bf16_to_f32(jssa.project_keys(keys, M))
    kf = bf16_to_f32(keys)
    for j in range(3):
        for i in range(r):
            exact = sum(Fraction(float(M[i, t])) * Fraction(float(kf[j, t])) for t in range(d))
            assert got[j, i] == np.float32(_exact_round_bf16(exact)), (j, i)


def test_identical_rows_get_identical_scores():
    rng = np.random.default_rng(5)
    row = _bf16(rng.standard_normal(32))
    kproj = np.tile(row, (1000, 1))
    q_hat = rng.standard_normal(32).astype(np.float32)
    s = jssa.score_positions(q_hat, kproj)
    assert np.all(s.view(np.uint32) == s.view(np.uint32)[0])
