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


# ---------------------------------------------------------------------------- fp8
# OCP FP8 E4M3 ("E4M3FN"): 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits;
# exponent 0 holds subnormals (fraction/8 * 2^-6); there are no infinities and only
# the all-ones exponent-and-fraction pattern (0x7F / 0xFF) is NaN, so the largest
# finite magnitude is 1.75 * 2^8 = 448. The projected scoring cache in this format
# is written unscaled and saturating: magnitudes beyond 448 store as 448.
FP8_MAX = 448.0
FP8_MIN_QUANTUM_EXP = -9      # subnormal step: 2^-3 * 2^-6


def fp8e4m3_to_f32(bits) -> np.ndarray:
    """Exact decoding of E4M3 bit patterns (uint8) to fp32; NaN patterns give NaN."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m, -9), np.ldexp(1.0 + m / 8.0, e - 7))
    val = sign * mag
    val = np.where((e == 15) & ((b & 0x7) == 7), np.nan, val)
    return val.astype(np.float32)


def round_to_fp8e4m3(x) -> np.ndarray:
    """Round real values (fp64 or fp32) to E4M3 in one step: nearest, ties to even,
    saturating at +-448; NaN gives 0x7F. Returns uint8 bit patterns.

    Method: as for bf16, x / quantum is an exact power-of-two scaling with quantum
    2^(e-4) for x = m * 2^e (0.5 <= |m| < 1; 4 significant bits), never below the
    subnormal step 2^-9; rint() rounds half to even. The rounded magnitude is then
    clamped to 448 and re-encoded field by field."""
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    xs = np.where(nan, 0.0, np.clip(x, -FP8_MAX, FP8_MAX))
    _, e = np.frexp(xs)
    qexp = np.maximum(e - 4, FP8_MIN_QUANTUM_EXP)
    r = np.minimum(np.abs(np.ldexp(np.rint(np.ldexp(xs, -qexp)), qexp)), FP8_MAX)
    sign = np.signbit(xs).astype(np.int64) << 7
    sub = r < 2.0 ** -6
    fexp = np.floor(np.log2(np.where(r > 0, r, 1.0))).astype(np.int64)
    frac_n = np.rint((np.ldexp(np.where(sub, 1.0, r), -np.where(sub, 0, fexp)) - 1.0) * 8.0).astype(np.int64)
    code_n = ((fexp + 7) << 3) | frac_n
    code_s = np.rint(np.ldexp(r, 9)).astype(np.int64)
    code = np.where(sub, code_s, code_n) | sign
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------- fp16
# IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits;
# largest finite 65504, smallest subnormal 2^-24.
FP16_MAX = 65504.0
FP16_MIN_QUANTUM_EXP = -24


def fp16_to_f32(bits) -> np.ndarray:
    """Exact decoding of binary16 bit patterns (uint16) to fp32, from the format
    definition: (-1)^s * 2^(e-15) * 1.f for normals, 2^-14 * 0.f for subnormals."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b & 0x8000, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    val = np.where(e == 0, np.ldexp(f, -24), np.ldexp(1024.0 + f, e - 25))
    val = np.where(e == 31, np.where(f == 0, np.inf, np.nan), val)
    return (sign * val).astype(np.float32)


def round_to_fp16(x) -> np.ndarray:
    """Round real values to binary16 in one step, ties to even; values that round
    above 65504 become infinity (IEEE overflow). Returns uint16 bit patterns.
    Same method as round_to_bf16 with 11 significant bits and quantum >= 2^-24."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    qexp = np.maximum(e - 11, FP16_MIN_QUANTUM_EXP)
    with np.errstate(over="ignore", invalid="ignore"):
        r = np.ldexp(np.rint(np.ldexp(x, -qexp)), qexp)
    nan = np.isnan(x)
    r = np.where(nan, 0.0, r)
    mag = np.abs(r)
    exp_field = np.zeros(r.shape, dtype=np.int64)
    frac = np.zeros(r.shape, dtype=np.int64)
    normal = mag >= 2.0 ** -14
    _, re = np.frexp(np.where(normal, mag, 1.0))
    exp_field = np.where(normal, re - 1 + 15, 0)
    frac = np.where(normal, np.rint(np.ldexp(np.where(normal, mag, 0.0), -(re - 1) + 10)) - 1024,
                    np.rint(np.ldexp(mag, 24)))
    over = mag > FP16_MAX
    bits = (exp_field << 10) | frac.astype(np.int64)
    bits = np.where(over, 0x7C00, bits)
    bits = bits | (np.signbit(x).astype(np.int64) << 15)
    bits = np.where(nan, 0x7E00, bits)
    return bits.astype(np.uint16)
