"""Number formats used by the path: MXFP4 (E2M1 + E8M0), FP8 E4M3, bf16.

The pages name the formats only: routed experts are stored as MXFP4 [ic §three
scalpels; card §method #1] and the LM head is turned into FP8 when it is built
[news §where the speed comes from; card §method #2].  The bit encodings are the
public OCP definitions:

* E2M1 [MX §5.3.3]: 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent 0 is
  subnormal (0 or 0.5); no Inf/NaN.  Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.
* E8M0 [MX §5.4.1]: unsigned 8-bit power of two 2^(b-127); 0xFF is NaN.
* MXFP4 block [MX §5.2]: 32 E2M1 elements share one E8M0 scale.  Memory
  packing (not fixed by MX; the reading adopted here): codes [N][K/2] bytes with
  the LOW nibble holding the even k, scales [N][K/32] row-major.
* E4M3 [OFP8 §4]: 1 sign, 4 exponent (bias 7), 3 mantissa; exponent 0 is
  subnormal (m * 2^-9); S.1111.111 is NaN; no Inf; largest finite 448.
* bf16: IEEE binary32 with the low 16 bits dropped; rounding is to nearest,
  ties to even.

Parity status: every function here is pinned (tests/test_oracle_formats.py):
E2M1 against the MX value table (golden fixture), E8M0 and E4M3 decode against
torch's float8_e8m0fnu / float8_e4m3fn decoders over all 256 codes, E4M3
encode against hand-picked midpoints and saturation cases plus torch's cast
for in-range values, bf16 rounding against torch's float32->bfloat16 cast,
MXFP4 packing against a hand-worked fixture.
"""

import numpy as np


def e2m1_value(code):
    """Value of 4-bit E2M1 codes (any integer array, only the low 4 bits used)."""
    c = np.asarray(code).astype(np.int64) & 0xF
    sign = (c >> 3) & 1
    exp = (c >> 1) & 3
    man = c & 1
    # exponent field 0: subnormal, man * 2^(1-bias) * 0.5 with bias 1 -> man * 0.5
    sub = man * 0.5
    # exponent field e > 0: 2^(e-1) * (1 + man/2)
    nor = np.power(2.0, exp - 1) * (1.0 + man / 2.0)
    mag = np.where(exp == 0, sub, nor)
    return np.where(sign == 1, -mag, mag).astype(np.float64)


def e8m0_value(code):
    """Value of E8M0 scale bytes: 2^(b-127); b = 255 encodes NaN."""
    b = np.asarray(code).astype(np.int64)
    v = np.power(2.0, b - 127)
    return np.where(b == 255, np.nan, v)


def mxfp4_dequant(codes, scales):
    """Dense float64 matrix [N][K] of an MXFP4 matrix.

    codes  uint8 [N][K/2], low nibble = element 2j, high nibble = element 2j+1
    scales uint8 [N][K/32], one E8M0 scale per 32 consecutive elements of a row
    Element (n, k) = e2m1(nibble(n, k)) * e8m0(scales[n][k // 32]).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    n, half_k = codes.shape
    k = 2 * half_k
    assert scales.shape == (n, k // 32), "one scale per 32 elements"
    lo = codes & 0x0F
    hi = codes >> 4
    nib = np.empty((n, k), dtype=np.uint8)
    nib[:, 0::2] = lo
    nib[:, 1::2] = hi
    elem = e2m1_value(nib)
    scale = np.repeat(e8m0_value(scales), 32, axis=1)
    return elem * scale


def e4m3_value(code):
    """Value of OCP E4M3 (FN) codes; 0x7F and 0xFF are NaN."""
    c = np.asarray(code).astype(np.int64) & 0xFF
    sign = (c >> 7) & 1
    exp = (c >> 3) & 0xF
    man = c & 7
    sub = man * 2.0 ** -9                      # 2^(1-7) * man/8
    nor = np.power(2.0, exp - 7) * (1.0 + man / 8.0)
    mag = np.where(exp == 0, sub, nor)
    mag = np.where((exp == 15) & (man == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


# The 127 non-negative finite E4M3 values, indexed by code 0x00..0x7E; they are
# strictly increasing in the code.
_E4M3_POS = e4m3_value(np.arange(0x7F))
E4M3_MAX = 448.0


def e4m3_encode_rne_sat(v):
    """E4M3 code of each float32 value: nearest finite value, ties to the even
    code, magnitudes above 448 saturate to 448, the sign (also of -0.0) kept.

    This is the rounding a hardware conversion to E4M3 in round-to-nearest-even
    saturating mode performs; it is written here as a search over the value
    table rather than as bit manipulation.
    """
    v = np.asarray(v, dtype=np.float32)
    assert not np.isnan(v).any(), "NaN is outside the input domain"
    a = np.abs(v).astype(np.float64)
    a = np.minimum(a, E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")      # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    exact = _E4M3_POS[hi] == a
    mid = (_E4M3_POS[lo] + _E4M3_POS[hi]) / 2.0           # exact in float64
    pick_hi = (a > mid) | ((a == mid) & (hi % 2 == 0))
    code = np.where(exact, hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    neg = np.signbit(v)
    return np.where(neg, code | 0x80, code).astype(np.uint8)


def bf16_round(y):
    """Round float64 values to the nearest bf16 value (ties to even).

    Returns float64 holding bf16-exact values.  Domain: 0 or normal bf16
    magnitudes (2^-126 .. below 2^128); the path never leaves it.
    """
    y = np.asarray(y, dtype=np.float64)
    m, e = np.frexp(y)                  # y = m * 2^e, 0.5 <= |m| < 1
    r = np.rint(m * 256.0)              # 8 significant bits, half to even
    return np.ldexp(r, e - 8)


def bf16_bits(v):
    """uint16 bit pattern of bf16-exact values."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(bits):
    """float64 value of uint16 bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
