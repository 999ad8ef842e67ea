"""Pins for the oracle's top-k: brute force over all subsets on tiny inputs, plus
invariants. Ranking rule: larger score first, ties to the lower position, NaN last."""
import itertools

import numpy as np

from oracle.jssa import select_topk


def _brute(scores, k):
    """Max-sum subset of size min(k, n); among equal sums the lexicographically
    smallest sorted index tuple (itertools.combinations yields that order)."""
    n = len(scores)
    kk = min(k, n)
    best, best_sum = None, None
    for comb in itertools.combinations(range(n), kk):
        tot = sum(int(scores[i]) for i in comb)
        if best_sum is None or tot > best_sum:
            best, best_sum = comb, tot
    return list(best) + [-1] * (k - kk)


def test_brute_force_all_subsets_with_ties():
    rng = np.random.default_rng(0)
    for n in range(1, 10):
        for _ in range(12):
            s = rng.integers(-2, 3, size=n).astype(np.float32)   # many exact ties
            for k in range(1, n + 3):
                assert list(select_topk(s, k)) == _brute(s, k), (s, k)


def test_signed_zero_ties_and_nan_last():
    s = np.array([0.0, -0.0, 0.0, -0.0], dtype=np.float32)
    assert list(select_topk(s, 2)) == [0, 1]
    s = np.array([np.nan, -np.inf, np.nan, -5.0], dtype=np.float32)
    assert list(select_topk(s, 1)) == [3]
    assert list(select_topk(s, 2)) == [1, 3]
    assert list(select_topk(s, 3)) == [0, 1, 3]          # then NaNs, lower position first
    s = np.array([np.inf, 1.0, np.inf], dtype=np.float32)
    assert list(select_topk(s, 2)) == [0, 2]


def test_padding_and_degenerate_sizes():
    assert list(select_topk(np.zeros(0, np.float32), 3)) == [-1, -1, -1]
    assert list(select_topk(np.array([3.0], np.float32), 4)) == [0, -1, -1, -1]


def test_permutation_equivariance_and_scale_invariance():
    rng = np.random.default_rng(1)
    s = rng.standard_normal(5000).astype(np.float32)
    k = 300
    base = select_topk(s, k)
    perm = rng.permutation(5000)
    moved = select_topk(s[perm], k)
    assert np.array_equal(np.sort(perm[moved]), base)
    for c in (0.25, 4.0, 1024.0):
        assert np.array_equal(select_topk(s * np.float32(c), k), base)
    # every selected score >= every unselected score
    mask = np.zeros(5000, bool)
    mask[base] = True
    assert s[mask].min() >= s[~mask].max()


def test_duplicated_values_take_lowest_positions():
    s = np.full(1000, 2.5, dtype=np.float32)
    s[[10, 500, 900]] = 7.0
    idx = select_topk(s, 8)
    assert list(idx) == [0, 1, 2, 3, 4, 10, 500, 900]
