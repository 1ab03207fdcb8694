"""Number formats, decoded from their bit definitions and rounded by definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Every decoder returns float64, which holds every value of these formats
exactly.  Every encoder rounds a float64 value to nearest, ties to even, with
the overflow rule of the target format, by scaling the value onto the target's
quantum grid (a power of two, so the scaling is exact in float64) and rounding
there with ``numpy.rint`` (ties to even).
"""

from fractions import Fraction

import numpy as np

# ---------------------------------------------------------------------------
# E4M3 (OCP "e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits,
# no infinities, S.1111.111 is NaN, largest finite magnitude 448.
# [NVFP4 card, "What is in the file": FP8 objects are e4m3fn with a row scale]
# [FP8 card, introduction: the text tower keeps E4M3 codes]
# ---------------------------------------------------------------------------


def e4m3_fraction(code):
    """Exact value of one E4M3 code as a Fraction (None for NaN)."""
    code = int(code) & 0xFF
    sign = -1 if code >> 7 else 1
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return None
    if exp == 0:                       # subnormal: 0.mmm x 2^(1-7)
        return sign * Fraction(man, 8) * Fraction(1, 2 ** 6)
    return sign * (1 + Fraction(man, 8)) * (Fraction(2) ** (exp - 7))


def _build_e4m3_table():
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        v = e4m3_fraction(c)
        if v is None:
            t[c] = np.nan
        elif v == 0:
            t[c] = -0.0 if c >> 7 else 0.0
        else:
            t[c] = float(v)            # exact: 4 significant bits
    return t


E4M3_TABLE = _build_e4m3_table()
E4M3_MAX = 448.0


def e4m3_decode(codes):
    """uint8 array of E4M3 codes -> float64 values (exact)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


# ---------------------------------------------------------------------------
# UE8M0: an unsigned 8-bit exponent, value 2^(b-127).
# [MXFP8 card, "How it was built", item 1]
# Reading: b = 255 is NaN (the OCP MX convention); the page gives only the
# formula, which covers 0..254.
# ---------------------------------------------------------------------------


def ue8m0_decode(b):
    b = np.asarray(b, dtype=np.int64)
    out = np.ldexp(1.0, (b - 127).astype(np.int64))
    return np.where(b == 255, np.nan, out)


# ---------------------------------------------------------------------------
# BF16 and IEEE binary16 decoders, from the field definitions.
# ---------------------------------------------------------------------------


def _decode_binary(bits, ebits, mbits):
    bits = np.asarray(bits, dtype=np.int64)
    bias = (1 << (ebits - 1)) - 1
    sign = np.where((bits >> (ebits + mbits)) & 1, -1.0, 1.0)
    e = (bits >> mbits) & ((1 << ebits) - 1)
    m = (bits & ((1 << mbits) - 1)).astype(np.float64)
    normal = np.ldexp(1.0 + m / (1 << mbits), e - bias)
    sub = np.ldexp(m / (1 << mbits), 1 - bias)
    val = np.where(e == 0, sub, normal)
    top = (1 << ebits) - 1
    val = np.where(e == top, np.where(m == 0, np.inf, np.nan), val)
    return sign * val


def bf16_decode(u16):
    """BF16 bit patterns (uint16) -> float64: 1 sign, 8 exponent (bias 127), 7 mantissa."""
    return _decode_binary(u16, 8, 7)


def f16_decode(u16):
    """IEEE binary16 bit patterns (uint16) -> float64: 1 sign, 5 exponent (bias 15), 10 mantissa."""
    return _decode_binary(u16, 5, 10)


def f32_decode(u32):
    return _decode_binary(u32, 8, 23)


# ---------------------------------------------------------------------------
# Round to nearest, ties to even, onto a binary floating-point grid.
# ---------------------------------------------------------------------------


def round_rne(x, p, emin, max_finite, saturate):
    """Round float64 values to a binary format with p significand bits.

    p: significand bits including the implicit one; emin: exponent of the
    smallest normal binade; max_finite: largest finite magnitude.
    Overflow: to +-max_finite if ``saturate`` else to +-inf (IEEE: a value
    rounds to infinity when it reaches max_finite plus half its ulp).
    NaN stays NaN.  The sign of zero is kept.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    with np.errstate(invalid="ignore", over="ignore"):
        _, e = np.frexp(ax)                    # ax in [2^(e-1), 2^e)
        lead = np.maximum(e - 1, emin)         # binade of the leading bit
        qexp = lead - (p - 1)                  # exponent of one unit in the last place
        r = np.ldexp(np.rint(np.ldexp(ax, -qexp)), qexp)
        over = r > max_finite
        r = np.where(over, max_finite if saturate else np.inf, r)
        r = np.where(np.isinf(ax), max_finite if saturate else np.inf, r)
        r = np.where(np.isnan(ax), np.nan, r)
    return np.copysign(r, x)


BF16_MAX = float((2 - Fraction(1, 2 ** 7)) * 2 ** 127)
F16_MAX = 65504.0
F32_MAX = float((2 - Fraction(1, 2 ** 23)) * 2 ** 127)


def round_bf16(x):
    return round_rne(x, 8, -126, BF16_MAX, saturate=False)


def round_f16(x):
    return round_rne(x, 11, -14, F16_MAX, saturate=False)


def round_f32(x):
    """Round float64 to the nearest float32 value (ties to even), as float64."""
    return round_rne(x, 24, -126, F32_MAX, saturate=False)


def round_e4m3_sat(x):
    """E4M3 RNE with saturation: |x| beyond 448 goes to +-448; NaN stays NaN."""
    return round_rne(x, 4, -6, E4M3_MAX, saturate=True)


def f32_div(a, b):
    """IEEE float32 division of float32-representable a by b.

    The float64 quotient is rounded to float32; double rounding cannot change
    a correctly rounded quotient because 53 >= 2*24 + 2.
    """
    with np.errstate(divide="ignore", invalid="ignore"):
        return round_f32(np.asarray(a, np.float64) / np.asarray(b, np.float64))


# ---------------------------------------------------------------------------
# Values -> bit patterns (for values already on the target grid).
# ---------------------------------------------------------------------------

_E4M3_POS = E4M3_TABLE[:127]          # codes 0x00..0x7E: increasing, finite


def e4m3_bits(v):
    """E4M3-representable float64 values (or NaN) -> uint8 codes, sign of zero kept."""
    v = np.asarray(v, dtype=np.float64)
    av = np.abs(v)
    idx = np.searchsorted(_E4M3_POS, np.where(np.isnan(av), 0.0, av))
    idx = np.minimum(idx, 126)
    if not np.all(np.isnan(av) | (_E4M3_POS[idx] == av)):
        raise ValueError("value not representable in E4M3")
    code = idx.astype(np.uint8) | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(av), np.uint8(0x7F), code).astype(np.uint8)


def bf16_bits(v):
    """BF16-representable float64 values -> uint16 bit patterns."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)   # exact for representable values
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def f32_bits(v):
    return np.asarray(v, dtype=np.float64).astype(np.float32).view(np.uint32)


def encode_e4m3(x):
    """float64 -> E4M3 code by RNE with saturation (NaN -> 0x7F)."""
    return e4m3_bits(round_e4m3_sat(x))


def encode_bf16(x):
    """float64 -> BF16 bits by RNE (overflow to infinity)."""
    r = round_bf16(x)
    return np.where(np.isnan(r), np.uint16(0x7FC0), bf16_bits(np.where(np.isnan(r), 0.0, r))).astype(np.uint16)
