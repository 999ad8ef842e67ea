"""Pins of the oracle's FP8 (OCP E4M3) scoring-cache format against an independent
implementation (torch.float8_e4m3fn) and the format's definition."""
import numpy as np
import torch

from oracle import jssa
from oracle.numerics import FP8_MAX, fp8e4m3_to_f32, round_to_fp8e4m3


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def _torch_encode(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine, ref = fp8e4m3_to_f32(codes), _torch_decode(codes)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.array_equal(mine[~np.isnan(mine)], ref[~np.isnan(ref)])
    assert np.sum(np.isnan(mine)) == 2                       # 0x7F and 0xFF only
    assert fp8e4m3_to_f32(np.uint8(0x7E)) == FP8_MAX         # largest finite
    assert fp8e4m3_to_f32(np.uint8(0x01)) == 2.0 ** -9       # smallest subnormal
    assert fp8e4m3_to_f32(np.uint8(0x08)) == 2.0 ** -6       # smallest normal


def test_encode_round_trip_and_torch_rne():
    codes = np.arange(256, dtype=np.uint8)
    vals = fp8e4m3_to_f32(codes)
    ok = ~np.isnan(vals)
    back = round_to_fp8e4m3(vals[ok])
    # every finite code decodes and re-encodes to itself (-0 keeps its sign)
    assert np.array_equal(back, codes[ok])
    # random values inside the finite range, and every exact midpoint between
    # neighbouring positive codes (ties to even), against torch's conversion
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(50000) * 3, rng.standard_normal(5000) * 100,
                        rng.standard_normal(5000) * 1e-3]).astype(np.float32)
    pos = np.sort(vals[ok & (vals > 0)].astype(np.float64))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)   # exact in fp32
    x = np.concatenate([x, mids, -mids])
    x = x[np.abs(x) <= FP8_MAX]
    assert np.array_equal(round_to_fp8e4m3(x), _torch_encode(x))


def test_saturation_nan_and_signed_zero():
    out = round_to_fp8e4m3(np.array([449.0, 463.9, 464.0, 1e9, np.inf, -np.inf, -500.0, np.nan, 0.0, -0.0]))
    assert list(out) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0x00, 0x80]


def test_fp8_scoring_uses_decoded_values():
    rng = np.random.default_rng(1)
    kp = rng.integers(0, 256, size=(50, 32)).astype(np.uint8)
    kp[kp == 0x7F] = 0x7E
    kp[kp == 0xFF] = 0xFE
    q = rng.standard_normal(32).astype(np.float32)
    s = jssa.score_positions(q, kp, "fp8")
    ref = (fp8e4m3_to_f32(kp).astype(np.float64) @ q.astype(np.float64)).astype(np.float32)
    assert np.array_equal(s, ref)
    # a key projected to fp8 is the fp64 projection rounded once
    k = (rng.standard_normal((20, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    M = np.linalg.qr(rng.standard_normal((128, 32)))[0].T.astype(np.float32)
    pk = jssa.project_keys(k, M, "fp8")
    exact = (k.astype(np.uint32) << 16).view(np.float32).astype(np.float64) @ M.astype(np.float64).T
    assert np.array_equal(pk, round_to_fp8e4m3(exact))
