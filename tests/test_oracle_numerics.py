"""Pins for the oracle's bf16 conversions against the format definition and torch."""
import numpy as np
import torch

from oracle.numerics import bf16_to_f32, round_to_bf16


def _torch_rne(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(x32.astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_widening_is_exact_and_round_trips():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = bf16_to_f32(allbits)
    finite = np.isfinite(f)
    # every finite bf16 value is an fp32 whose low 16 bits are zero
    assert np.all((f.view(np.uint32)[finite] & 0xFFFF) == 0)
    back = round_to_bf16(f[finite])
    assert np.array_equal(back, allbits[finite])


def test_matches_torch_rne_from_fp32():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(3.0),
        rng.standard_normal(20000).astype(np.float32) * np.float32(1e30),
        rng.standard_normal(20000).astype(np.float32) * np.float32(1e-38),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 3.4028235e38], dtype=np.float32),
    ])
    # exact ties at bf16 precision: low 16 bits == 0x8000
    ties = (rng.integers(0, 2**31, 5000, dtype=np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32)])
    x = x[np.isfinite(x) | np.isinf(x)]
    assert np.array_equal(round_to_bf16(x), _torch_rne(x))


def test_ties_to_even_and_single_rounding():
    q = 2.0 ** -7                   # bf16 quantum on [1, 2)
    cases = {
        1.0 + q / 2: 1.0,            # tie, 1.0 has an even significand
        1.0 + 1.5 * q: 1.0 + 2 * q,  # tie between odd and even -> even
        1.0 + q / 2 + 2.0 ** -40: 1.0 + q,   # above the tie only in fp64: one rounding step
        -(1.0 + q / 2): -1.0,
    }
    for x, want in cases.items():
        got = bf16_to_f32(round_to_bf16(np.array([x])))[0]
        assert got == np.float32(want), (x, got, want)


def test_subnormals_and_overflow():
    tiny = 2.0 ** -133
    got = round_to_bf16(np.array([tiny, tiny / 2, 1.5 * tiny, 3 * tiny / 2 * 1.0000001, 2.0 ** 128, -2.0 ** 129]))
    assert got[0] == 0x0001
    assert got[1] == 0x0000         # tie with 0 -> even (0)
    assert got[2] == 0x0002         # tie between 1 and 2 quanta -> even (2)
    assert got[3] == 0x0002
    assert got[4] == 0x7F80         # +inf
    assert got[5] == 0xFF80         # -inf
    nan = round_to_bf16(np.array([np.nan]))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x007F) != 0
