"""The GEMM1 epilogue's division-free MX scale code (host check).

An MX group's scale is pow2_at_least(amax / 448) with the quotient formed in
fp32 ([MegaMoE] §3.5, the epilogue that fuses SwiGLU and the
re-quantisation).  The MXFP4 GEMM1
epilogue reads the e8m0 code straight from amax's bits instead: for
amax = 1.m x 2^(E-127) with E in [10, 254] the code is E - 8, plus one when
1.m > 1.75 (mantissa field above 0x600000).  That identity holds because the
fp32 quotient rounds to at most 2^e exactly when amax <= 448 x 2^e (448 is
1.75 x 2^8, and the rounding boundary just above 448 x 2^e lies below the
next fp32 value).  This test checks it against the oracle's pow2_at_least of
the fp32 quotient over every mantissa of several exponents (the identity does
not depend on the exponent inside that range), both ends of the range
included, and that the scaled values then stay within +-448 (the epilogue
leaves out the clamp).
"""

import numpy as np
import pytest

from oracle import formats as fm


def _code_from_quotient(a32):
    q = (a32 / np.float32(448.0)).astype(np.float32)  # fp32 division, correctly rounded
    scale = fm.pow2_at_least(q.astype(np.float64))
    return np.log2(scale).astype(np.int64) + 127


def _code_from_bits(a32):
    u = a32.view(np.uint32).astype(np.int64)
    E = (u >> 23) & 0xFF
    return E - 8 + ((u & 0x7FFFFF) > 0x600000)


@pytest.mark.parametrize("E", [10, 11, 64, 127, 128, 200, 253, 254])
def test_mx_code_from_bits_equals_fp32_quotient_code(E):
    mant = np.arange(1 << 23, dtype=np.uint32)
    a = ((np.uint32(E) << 23) | mant).view(np.float32)
    got = _code_from_bits(a)
    want = _code_from_quotient(a)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"E={E}: first mismatch at mantissa {hex(int(mant[bad[0]]))}"
    # |v| <= amax <= 448 x 2^(code - 127): the scaled values need no clamp
    scaled = a.astype(np.float64) / np.ldexp(1.0, (got - 127).astype(np.int64))
    assert np.all(scaled <= 448.0)
