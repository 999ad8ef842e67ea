"""Pins of the block-sparse oracle (block keys, INT4 selector cache, block scores,
block selection) against hand-worked values, numpy's binary16 conversion, closed
forms and brute force."""
import itertools

import numpy as np
import pytest

from oracle import blocksparse as bs
from oracle import jssa
from oracle.numerics import bf16_to_f32, fp16_to_f32, round_to_bf16, round_to_fp16


def _bf16(x):
    return round_to_bf16(np.asarray(x, dtype=np.float64))


def test_fp16_rounding_matches_numpy_binary16():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000) * 10.0 ** rng.integers(-9, 6, 200000)
    x = np.concatenate([x, [0.0, -0.0, 65504.0, 65519.9, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14]])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(round_to_fp16(x), ref)
    allbits = np.arange(65536, dtype=np.uint16)
    dec = fp16_to_f32(allbits)
    want = allbits.view(np.float16).astype(np.float32)
    same = (dec.view(np.uint32) == want.view(np.uint32)) | (np.isnan(dec) & np.isnan(want))
    assert np.all(same)


def test_block_keys_hand_worked():
    # block of 4 rows 1, 2, 3, 4 -> mean 2.5 (exact); block of 2 rows 1 and 1 + 2^-7
    # -> mean 1 + 2^-8, a bf16 tie that rounds to the even neighbour 1.0
    K = _bf16(np.array([[1.0], [2.0], [3.0], [4.0]]) * np.ones((1, 4)))
    kc = bs.block_keys(K, 4, 4)
    assert kc.shape == (1, 4) and np.all(bf16_to_f32(kc) == 2.5)
    K2 = _bf16(np.array([[1.0], [1.0 + 2 ** -7], [3.0], [3.0]]) * np.ones((1, 4)))
    kc2 = bs.block_keys(K2, 4, 2)
    assert np.all(bf16_to_f32(kc2[0]) == 1.0) and np.all(bf16_to_f32(kc2[1]) == 3.0)
    # only complete blocks get a key
    assert bs.block_keys(K2, 3, 2).shape == (1, 4)
    assert bs.block_keys(K2, 1, 2).shape == (0, 4)


def test_block_keys_of_identical_rows_are_the_row():
    rng = np.random.default_rng(1)
    row = _bf16(rng.standard_normal(128))
    K = np.tile(row, (64 * 3, 1))
    kc = bs.block_keys(K, 64 * 3 - 1, 64)
    assert kc.shape == (2, 128) and np.array_equal(kc[0], row) and np.array_equal(kc[1], row)


def test_int4_scale_and_codes_hand_worked():
    # absmax 7 -> scale exactly 1: codes are the values rounded half to even
    vals = np.array([7.0, 3.5, 2.5, -7.0, 0.5, -0.5, 1.5, -2.5] * 8 + [0.0] * 64)
    kc = _bf16(vals)[None]
    codes, scales = bs.int4_quantize(kc)
    assert np.all(fp16_to_f32(scales[0]) == [1.0, 0.0])
    assert list(codes[0, :8]) == [7, 4, 2, -7, 0, 0, 2, -2]
    assert np.all(codes[0, 64:] == 0)                   # all-zero group: scale 0, codes 0
    # absmax 0.6875: scale = binary16(0.6875f / 7) = 1609 * 2^-14
    g = np.full(64, 0.0)
    g[:4] = [0.6875, -0.34375, 0.046875, 0.0]
    codes, scales = bs.int4_quantize(_bf16(np.concatenate([g, g]))[None])
    assert fp16_to_f32(scales[0, 0]) == 1609 * 2.0 ** -14
    s = 1609 * 2.0 ** -14
    assert list(codes[0, :4]) == [7, int(np.rint(-0.34375 / s)), int(np.rint(0.046875 / s)), 0] == [7, -4, 0, 0]


def test_int4_against_binary16_library_and_error_bound():
    rng = np.random.default_rng(2)
    kc = _bf16(rng.standard_normal((50, 128)) * rng.uniform(0.01, 10, (50, 1)))
    codes, scales = bs.int4_quantize(kc)
    x = bf16_to_f32(kc).reshape(50, 2, 64)
    absmax = np.abs(x).max(axis=2)
    want_scale = (absmax / np.float32(7)).astype(np.float32).astype(np.float16)
    assert np.array_equal(scales, want_scale.view(np.uint16))
    s = want_scale.astype(np.float32)
    want_codes = np.clip(np.rint((x / s[:, :, None]).astype(np.float32)), -7, 7)
    assert np.array_equal(codes.reshape(50, 2, 64), want_codes.astype(np.int8))
    deq = bs.int4_dequantize(codes, scales).reshape(50, 2, 64)
    # within half a step, except where the fp16 rounding of the scale pushed |x| past 7 steps
    err = np.abs(deq - x)
    inside = np.abs(x) <= 7 * s[:, :, None]
    assert np.all(err[inside] <= s[:, :, None].repeat(64, axis=2)[inside] / 2 * (1 + 1e-6))
    assert np.all(err <= absmax[:, :, None] * 0.08)


def test_int4_packing():
    codes = np.array([[1, -1, 7, -7, 0, -3]], dtype=np.int8)
    packed = bs.pack_int4(codes)
    assert list(packed[0]) == [0xF1, 0x97, 0xD0]
    allc = np.array([list(range(-7, 8)) + [0]], dtype=np.int8)
    assert np.array_equal(bs.unpack_int4(bs.pack_int4(allc)), allc)


def test_block_scores_closed_forms():
    rng = np.random.default_rng(3)
    q = _bf16(rng.standard_normal((8, 128)))
    kc = bf16_to_f32(_bf16(rng.standard_normal((37, 128))))
    s = bs.block_scores(q, kc, 0.125)
    assert abs(s.sum() - 8.0) < 1e-12                   # each head's softmax sums to 1
    # a common vector added to every block key shifts each head's logits uniformly
    shift = bf16_to_f32(_bf16(rng.standard_normal(128))).astype(np.float64)
    s2 = bs.block_scores(q, kc.astype(np.float64) + shift, 0.125)
    assert np.max(np.abs(s - s2)) < 1e-12
    # one head, two blocks whose logits differ by delta: scores are the logistic pair
    q1 = _bf16(np.concatenate([[1.0], np.zeros(127)]))[None]
    k2 = np.zeros((2, 128))
    k2[0, 0], k2[1, 0] = 2.0, -1.0
    s3 = bs.block_scores(q1, k2, 0.5)
    assert abs(s3[0] - 1 / (1 + np.exp(-1.5))) < 1e-15 and abs(s3[1] - 1 / (1 + np.exp(1.5))) < 1e-15


def test_forced_blocks():
    assert list(bs.forced_blocks(65536, 64, 1, 2)) == [0, 1022, 1023]
    assert list(bs.forced_blocks(65537, 64, 1, 2)) == [0, 1023, 1024]
    assert list(bs.forced_blocks(100, 64, 1, 2)) == [0, 1]
    assert list(bs.forced_blocks(0, 64, 1, 2)) == []


def _brute(s, n, block, k_blocks, n_init, n_local):
    forced = set(bs.forced_blocks(n, block, n_init, n_local))
    m = bs.complete_blocks(n, block)
    elig = [j for j in range(m) if j not in forced]
    room = k_blocks - len(forced)
    best, best_key = None, None
    for c in itertools.combinations(elig, min(room, len(elig))):
        key = (-sum(sorted(s[list(c)])), c)
        if best_key is None or key < best_key:
            best, best_key = c, key
    return sorted(list(forced) + list(best))


@pytest.mark.parametrize("seed", range(5))
def test_block_selection_brute_force(seed):
    rng = np.random.default_rng(seed)
    block = 4
    for n in range(0, 41, 3):
        nb = bs.total_blocks(n, block)
        m = bs.complete_blocks(n, block)
        s = rng.integers(0, 3, size=max(m, 1)).astype(np.float64)[:m]     # many ties
        for k_blocks in range(3, 8):
            got = bs.select_blocks(s, n, block, k_blocks, 1, 2)
            if nb <= k_blocks:
                assert list(got) == list(range(nb))
            else:
                assert list(got) == _brute(s, n, block, k_blocks, 1, 2), (n, k_blocks, s)


def test_whole_budget_is_dense_attention():
    rng = np.random.default_rng(4)
    n, block = 200, 16
    q = _bf16(rng.standard_normal((8, 32)))
    K = _bf16(rng.standard_normal((n, 32)))
    V = _bf16(rng.standard_normal((n, 32)))
    kc = bf16_to_f32(bs.block_keys(K, n, block))
    out, idx, blocks, _ = bs.decode_unit(q, K, V, kc, n, block, 13, 1, 2, 0.2)
    assert list(blocks) == list(range(13)) and list(idx[:n]) == list(range(n))
    ref = jssa.attend(q, K, V, np.arange(n), 0.2)
    assert np.max(np.abs(out - ref)) < 1e-12
