"""Exact decoders for the stored number formats, and the e4m3 quantiser.

Test infrastructure only (see ``oracle/__init__``).

Formats
-------
* bf16: the upper 16 bits of an IEEE binary32.  Hidden states and bf16
  expert weights ([Router] §2 "Why Engines Don't Round the Router": bf16
  activations and weights, fp32 logits and bias).
* E4M3FN (OCP 8-bit float, 4 exponent bits, bias 7, 3 mantissa bits, no
  infinities, S.1111.111 is NaN, largest finite 448).  448 as the largest
  FP8 value is used by the requantisation in [MegaMoE] §3.5; the fp8 block
  formats are those of [Kernels] "Combine, backward and low precision".
* E2M1 (OCP 4-bit float, 2 exponent bits, bias 1, 1 mantissa bit; finite
  magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) and E8M0 (a pure power of two
  2^(b-127), 255 is NaN): the MX formats of [MegaMoE] §1.1 (4-bit weights,
  one shared scale per 32 values).

Every decoder is written from the bit-field definition; the tests pin them
against independent sources (torch's float8_e4m3fn cast for every code, the
OCP value table for e2m1).
"""

import math

import numpy as np

E4M3_MAX = 448.0


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) -> exact float64 values."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(values):
    """float64 -> bf16 bits with round-to-nearest-even (via float32 first).

    Used only to build test inputs whose values are already exact bf16
    numbers; the oracle itself never rounds to bf16.
    """
    f = np.asarray(values, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return u.astype(np.uint16)


def e4m3_decode(codes):
    """OCP E4M3FN codes (uint8) -> float64 (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = (c & 0x7).astype(np.float64)
    normal = (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    subnormal = (man / 8.0) * 2.0 ** -6
    val = np.where(exp == 0, subnormal, normal)
    val = np.where((exp == 15) & (c & 0x7 == 7), np.nan, val)
    return sign * val


def e2m1_decode(nibbles):
    """OCP E2M1 4-bit codes (values 0..15) -> float64."""
    c = np.asarray(nibbles, dtype=np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    exp = (c >> 1) & 0x3
    man = (c & 0x1).astype(np.float64)
    normal = (1.0 + man / 2.0) * np.exp2(exp.astype(np.float64) - 1.0)
    subnormal = man / 2.0
    return sign * np.where(exp == 0, subnormal, normal)


def e8m0_decode(codes):
    """E8M0 scale codes (uint8) -> float64 powers of two (255 -> NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def unpack_fp4(packed, axis=-1):
    """Two e2m1 codes per byte along ``axis``: element 2j sits in the low
    nibble of byte j and element 2j+1 in the high nibble.  Returns the codes
    (not the values), with ``axis`` doubled in length."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = p & 0xF
    hi = p >> 4
    out = np.stack([lo, hi], axis=-1 if axis == -1 else axis + 1)
    shape = list(p.shape)
    shape[axis] *= 2
    return out.reshape(shape)


# Positive finite e4m3 magnitudes in code order (codes 0x00..0x7E); the
# code order is also the order of the values, so an even code has an even
# mantissa.
_E4M3_POS = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_round(values):
    """Round float64 values to the nearest E4M3FN value, ties to the even
    code, saturating at +-448 (no NaN is produced for finite input).

    Returned as float64 values on the e4m3 grid (the emulate mode needs the
    value, not the code)."""
    v = np.asarray(values, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")  # first grid >= a
    hi = np.minimum(hi, len(_E4M3_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    g_hi = _E4M3_POS[hi]
    g_lo = _E4M3_POS[lo]
    d_hi = g_hi - a
    d_lo = a - g_lo
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    pick_hi |= g_hi == a
    r = np.where(pick_hi, g_hi, g_lo)
    return np.copysign(r, v)


def pow2_at_least(v):
    """Smallest power of two >= v for v > 0 (float64, exact).  Takes a
    number (returns a float) or an array (returns an array)."""
    if np.ndim(v) == 0:
        v = float(v)
        if v <= 0.0:
            raise ValueError("pow2_at_least needs a positive argument")
        m, e = math.frexp(v)  # v = m * 2**e with 0.5 <= m < 1
        return math.ldexp(1.0, e - 1) if m == 0.5 else math.ldexp(1.0, e)
    v = np.asarray(v, dtype=np.float64)
    if np.any(v <= 0.0):
        raise ValueError("pow2_at_least needs positive arguments")
    m, e = np.frexp(v)
    return np.ldexp(1.0, e - (m == 0.5))
