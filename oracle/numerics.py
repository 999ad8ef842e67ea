"""bf16 <-> float conversions for the oracle, written from the format definition.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and the benchmark's
cpu_baseline leg may import anything under oracle/. It shares no code with the
HIP path.

bf16 is the upper half of an IEEE-754 binary32: 1 sign bit, 8 exponent bits and
7 stored fraction bits (8 significant bits for normal numbers). numpy has no
bf16 dtype, so bf16 tensors travel as uint16 bit patterns.
"""
from __future__ import annotations

import numpy as np

BF16_MIN_QUANTUM_EXP = -133   # smallest bf16 subnormal is 2^-133 (fp32 exponent range, 7 fraction bits)


def bf16_to_f32(bits) -> np.ndarray:
    """Exact widening: the bf16 pattern becomes the high 16 bits of an fp32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def round_to_bf16(x) -> np.ndarray:
    """Round real values (given as fp64 or fp32) to the nearest bf16, ties to even,
    in one rounding step. Returns uint16 bit patterns.

    Method: write x = m * 2^e with 0.5 <= |m| < 1 (frexp). A normal bf16 near x has
    8 significant bits, i.e. a quantum of 2^(e-8); below the normal range the
    quantum stays at 2^-133. x / quantum is an exact power-of-two scaling, rint()
    rounds it half-to-even, and the product is exact. Values that reach 2^128
    overflow to infinity. NaN maps to the canonical quiet NaN with x's sign.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    qexp = np.maximum(e - 8, BF16_MIN_QUANTUM_EXP)
    with np.errstate(over="ignore", invalid="ignore"):
        scaled = np.ldexp(x, -qexp)
        r = np.ldexp(np.rint(scaled), qexp)
        r = np.where(np.isfinite(x), r, x)
        f32 = r.astype(np.float32)            # exact: r has at most 8 significant bits
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if np.any(nan):
        sign = (np.signbit(x).astype(np.uint16) << np.uint16(15))
        bits = np.where(nan, sign | np.uint16(0x7FC0), bits).astype(np.uint16)
    return bits


def f32_round(x) -> np.ndarray:
    """Round real values held in fp64 to the nearest fp32 (ties to even; IEEE cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)
