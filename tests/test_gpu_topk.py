"""GPU top-k (sjsa_topk) against the oracle on planted scores: bit-exact index sets,
including exact ties, signed zeros, NaN and infinities, ragged lengths, and budgets
that exercise both the LDS path and the multi-pass fallback."""
import numpy as np
import pytest
import torch

import token_level_sparse_kv_amd as sj
from oracle.jssa import select_topk
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu


def _run(scores: np.ndarray, seq_len, k):
    B, H, stride = scores.shape
    s = torch.from_numpy(scores).cuda()
    sl = torch.tensor(seq_len, dtype=torch.int32, device="cuda")
    idx = sj.topk(s, sl, k)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for b in range(B):
        n = min(max(seq_len[b], 0), stride)
        for h in range(H):
            want = select_topk(scores[b, h, :n], k)
            assert np.array_equal(got[b, h], want), (b, h, n, k, np.flatnonzero(got[b, h] != want)[:10])


def _rng(seed):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("k", [1, 7, 100, 4096, 9999, 10000, 12000])
def test_random_scores(k):
    say(f"topk random k={k}")
    s = _rng(k).standard_normal((2, 3, 10000)).astype(np.float32)
    _run(s, [10000, 9973], k)


def test_heavy_ties_small_integers():
    say("topk integer ties")
    s = _rng(1).integers(-3, 4, size=(2, 2, 20000)).astype(np.float32)
    _run(s, [20000, 19999], 5000)
    _run(s, [20000, 17], 5)


def test_all_equal_fallback_path():
    say("topk all equal (fallback)")
    s = np.full((1, 2, 50000), 1.5, dtype=np.float32)
    s[0, 1, ::7] = 2.0
    _run(s, [50000], 3000)


def test_constant_row_takes_the_first_positions():
    # more equal keys than the lists hold: the crowded-bin check finds one key value
    say("topk constant row (crowded bin, one key)")
    s = np.full((2, 2, 50000), -0.75, dtype=np.float32)
    _run(s, [50000, 49999], 3000)
    _run(s, [50000, 20000], 16000)


def test_crowded_bin_of_one_key_below_other_keys():
    # 300 keys above a crowded bin whose keys are all equal: the threshold is that key
    say("topk crowded bin of one key, 300 keys above")
    s = np.full((1, 2, 40000), 1.0, dtype=np.float32)
    pos = _rng(6).choice(40000, 300, replace=False)
    s[0, 0, pos] = 3.0
    s[0, 1, pos] = _rng(7).uniform(2.0, 4.0, 300).astype(np.float32)
    _run(s, [40000], 1000)


def test_crowded_bin_of_distinct_keys():
    # 50000 keys in [1, 1.125): one first-digit bin (sign, exponent and three mantissa
    # bits), distinct low bits, with exact repeats: the two radix rounds resolve it
    say("topk crowded bin of distinct keys")
    rng = _rng(8)
    s = (1.0 + rng.integers(0, 1 << 17, size=(2, 2, 50000)) * np.float32(2.0 ** -20)).astype(np.float32)
    s[:, 1, ::2] = s[:, 1, 1::2]
    _run(s, [50000, 50000], 3000)
    _run(s, [50000, 45001], 20000)


def test_large_budget_fallback_path():
    say("topk large k (fallback)")
    s = _rng(2).standard_normal((1, 2, 100000)).astype(np.float32)
    _run(s, [100000], 20000)
    _run(s, [99999], 99990)


def test_signed_zero_nan_inf():
    say("topk specials")
    s = _rng(3).standard_normal((1, 4, 4096)).astype(np.float32)
    s[0, 0] = 0.0
    s[0, 0, 1::2] = -0.0
    s[0, 1, ::3] = np.nan
    s[0, 2, ::5] = -np.inf
    s[0, 2, 7] = np.inf
    s[0, 3] = np.nan
    s[0, 3, 100:110] = -np.inf
    for k in (1, 50, 2000, 4096):
        _run(s, [4096], k)


def test_empty_and_short_rows():
    say("topk empty/short")
    s = _rng(4).standard_normal((3, 2, 64)).astype(np.float32)
    _run(s, [0, 1, 64], 16)
    _run(s, [-5, 63, 1000], 64)


def test_duplicated_blocks_lower_position_wins():
    say("topk duplicates")
    base = _rng(5).standard_normal(1000).astype(np.float32)
    s = np.tile(base, 40)[None, None, :].copy()                      # every value appears 40 times
    _run(s, [40000], 777)
