"""Bit-level rounding of the oracle -- test infrastructure (see the package docstring).

Everything here is written from the number formats' definitions, not from any library cast:

  * A binary floating-point format with p significant bits (implicit bit included) and smallest
    normal exponent emin represents, for a value of magnitude in [2^e, 2^(e+1)), the multiples of
    2^(max(e, emin) - p + 1); below 2^emin the spacing stays 2^(emin - p + 1) (subnormals).
    Rounding is to the nearest such multiple, ties to the even multiple.
  * bfloat16: p = 8, emin = -126, overflow to +-infinity (binary32 with 16 mantissa bits dropped).
  * OCP FP8 E4M3 ("e4m3fn", the 8-bit float of the Wan 8-bit attention's PV product): 1 sign bit,
    4 exponent bits with bias 7, 3 mantissa bits; p = 4, emin = -6; no infinities, the codes
    S.1111.111 are NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.  Values beyond +-448
    are clamped to +-448 before rounding (a saturating conversion; the pages do not say how
    overflow is treated -- this is the reading taken).
  * int8 codes of the symmetric per-block quantisation: round(x * inv) with ties to even, clamped
    to [-127, 127] (the pages give int8 for Q and K in the 8-bit attention, "Wan模型是什么它能做什么"
    explainer, section 4.2, but not the rounding; round-half-even and the symmetric range are the
    reading taken).
"""

import numpy as np


def round_to_binary(x, sig_bits, emin):
    """Round float64 values to a binary format with ``sig_bits`` significant bits and smallest
    normal exponent ``emin`` (no overflow handling, no NaN handling).  Returns float64."""
    x = np.asarray(x, dtype=np.float64)
    _, E = np.frexp(x)                     # |x| = f * 2^E with f in [0.5, 1)
    e = np.maximum(E - 1, emin)            # exponent of the binade, floored at the normal range
    quantum = np.ldexp(np.ones_like(x), e - (sig_bits - 1))
    return np.round(x / quantum) * quantum  # np.round is round-half-to-even; x / quantum is exact


def bf16_round(x):
    """Round float32 (or float64 values exactly representable in float32) to bfloat16, ties to
    even.  Returns float32 arrays holding bfloat16 values."""
    x = np.asarray(x, dtype=np.float64)
    r = round_to_binary(np.where(np.isfinite(x), x, 0.0), 8, -126)
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, x), r)
    r = np.where(np.isfinite(x), r, x)
    return r.astype(np.float32)


E4M3_MAX = 448.0


def e4m3fn_round(x):
    """Saturating round to OCP e4m3fn values (clamp to +-448, then nearest, ties to even).
    Returns float64 holding e4m3fn values."""
    x = np.asarray(x, dtype=np.float64)
    c = np.clip(x, -E4M3_MAX, E4M3_MAX)
    r = round_to_binary(c, 4, -6)
    return np.where(np.isnan(x), np.nan, r)


def e4m3fn_decode(codes):
    """Value of each e4m3fn code (uint8) as float64; NaN for the codes S.1111.111."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    E = (c >> 3) & 0xF
    M = (c & 0x7).astype(np.float64)
    normal = (1.0 + M / 8.0) * np.ldexp(1.0, E - 7)
    subnormal = (M / 8.0) * 2.0 ** -6
    mag = np.where(E == 0, subnormal, normal)
    mag = np.where((E == 0xF) & (c & 0x7 == 0x7), np.nan, mag)
    return sign * mag


def e4m3fn_encode(values):
    """Code (uint8) of each value, which must already be an e4m3fn value (e.g. the output of
    ``e4m3fn_round``).  Negative zero keeps its sign bit (code 0x80)."""
    v = np.asarray(values, dtype=np.float64)
    if np.any(~np.isfinite(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("not an e4m3fn value")
    sign = np.signbit(v).astype(np.int64)
    a = np.abs(v)
    _, E = np.frexp(np.where(a > 0, a, 1.0))
    e = E - 1
    sub = (a > 0) & (e < -6)
    exp_field = np.where(sub | (a == 0), 0, e + 7)
    mant = np.where(sub, a / 2.0 ** -9, (a / np.ldexp(1.0, np.where(sub, 0, e)) - 1.0) * 8.0)
    mant = np.where(a == 0, 0.0, mant)
    if np.any(mant != np.round(mant)) or np.any((mant < 0) | (mant > 7)):
        raise ValueError("not an e4m3fn value")
    return ((sign << 7) | (exp_field << 3) | mant.astype(np.int64)).astype(np.uint8)


def int8_codes(x, inv):
    """Symmetric int8 codes: clamp(round_half_even(x * inv), -127, 127), with the product taken in
    float32 (x and inv are converted to float32 first).  Returns int8."""
    xf = np.asarray(x, dtype=np.float32)
    prod = (xf * np.float32(inv) if np.ndim(inv) == 0 else xf * np.asarray(inv, np.float32))
    prod = prod.astype(np.float32)
    return np.clip(np.rint(prod), -127, 127).astype(np.int8)
