"""Number formats used on the wire: bf16 input, FP8 E4M3 / E5M2 codes, packed INT4.

Test infrastructure only (see the package docstring).
"""

import numpy as np

F32 = np.float32

# E4M3 constants from the format definition ([FP8]; [TACO] Fig. 3 picks E4M3).
E4M3_BIAS = 7
E4M3_MAX = 448.0          # S.1111.110
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_MIN_SUBNORMAL = 2.0 ** -9
E4M3_NAN = 0x7F           # S.1111.111; the encoder below emits the positive one


def bf16_bits_to_f32(bits):
    """Widen bf16 bit patterns (uint16) to float32: the bits become the top half."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x):
    """Round float32 to bf16 (nearest, ties to even); NaN becomes 0x7FC0.

    Used for the bf16 output of the final decode and by nothing on the
    compression side.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), r).astype(np.uint16)


def decode_e4m3(codes):
    """Value of each E4M3 code, written out from the bit fields ([FP8]).

    sign s, exponent field e (4 bits, bias 7), mantissa m (3 bits):
    e == 0 -> (-1)^s * m * 2^-9 (subnormal); otherwise (-1)^s * (1 + m/8) * 2^(e-7);
    e == 15 and m == 7 -> NaN. There is no infinity.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - E4M3_BIAS))
    val = np.where(s == 1, -mag, mag)
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return val.astype(np.float32)


def encode_e4m3(v):
    """Round float32 values to E4M3 codes: nearest, ties to even, saturating.

    Reading (the pages name E4M3 in [TACO] Fig. 3 and bound its error in
    Eq. (3) but fix neither rounding nor overflow): round to nearest with ties
    to the even mantissa; magnitudes at or above 448 (including infinity)
    saturate to +-448; NaN encodes as 0x7F; the sign bit is kept for values
    that round to zero. Every scaling below is by a power of two, so the only
    rounding is the one ``np.rint`` performs.
    """
    v = np.asarray(v, dtype=np.float32)
    nan = np.isnan(v)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    a = np.minimum(np.abs(v.astype(np.float64)), E4M3_MAX)
    a = np.where(nan, 0.0, a)

    # subnormal range: a < 2^-6, step 2^-9; m == 8 lands on the smallest normal
    m_sub = np.rint(a * 512.0).astype(np.int64)

    # normal range: a = f * 2^E with f in [0.5, 1); exponent e = E - 1
    _, E = np.frexp(np.where(a > 0, a, 1.0))
    e = E.astype(np.int64) - 1
    m = np.rint(np.ldexp(a, (3 - e))).astype(np.int64) - 8      # in [0, 8]
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    code_norm = ((e + E4M3_BIAS) << 3) | m

    code = np.where(a < E4M3_MIN_NORMAL, m_sub, code_norm) | sign
    code = np.where(nan, E4M3_NAN, code)
    return code.astype(np.uint8)


# E5M2 constants from the format definition ([FP8]; [TACO] Fig. 3 sets E5M2
# beside E4M3): 5 exponent bits with bias 15, 2 mantissa bits, IEEE-style
# infinities and NaNs in the top exponent.
E5M2_BIAS = 15
E5M2_MAX = 57344.0        # S.11110.11
E5M2_MIN_NORMAL = 2.0 ** -14
E5M2_MIN_SUBNORMAL = 2.0 ** -16
E5M2_INF = 0x7C           # S.11111.00
E5M2_NAN = 0x7F           # S.11111.11; the encoder below emits the positive one


def decode_e5m2(codes):
    """Value of each E5M2 code, written out from the bit fields ([FP8]).

    sign s, exponent field e (5 bits, bias 15), mantissa m (2 bits):
    e == 0 -> (-1)^s * m * 2^-16 (subnormal); e == 31 -> +-inf (m == 0) or NaN;
    otherwise (-1)^s * (1 + m/4) * 2^(e-15).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 2) & 0x1F
    m = c & 3
    mag = np.where(e == 0, m * 2.0 ** -16, (1.0 + m / 4.0) * np.exp2(np.minimum(e, 30) - E5M2_BIAS))
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    val = np.where(s == 1, -mag, mag)
    return val.astype(np.float32)


def encode_e5m2(v):
    """Round float32 values to E5M2 codes: nearest, ties to even, saturating.

    The same reading as ``encode_e4m3`` (the pages fix neither rounding nor
    overflow): ties go to the even mantissa; finite magnitudes above 57344 and
    infinities saturate to +-57344 (no infinity is produced); NaN encodes as
    0x7F; the sign bit is kept for values that round to zero.
    """
    v = np.asarray(v, dtype=np.float32)
    nan = np.isnan(v)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    a = np.minimum(np.abs(v.astype(np.float64)), E5M2_MAX)
    a = np.where(nan, 0.0, a)

    # subnormal range: a < 2^-14, step 2^-16; m == 4 lands on the smallest normal
    m_sub = np.rint(a * 65536.0).astype(np.int64)

    # normal range: a = f * 2^E with f in [0.5, 1); exponent e = E - 1
    _, E = np.frexp(np.where(a > 0, a, 1.0))
    e = E.astype(np.int64) - 1
    m = np.rint(np.ldexp(a, (2 - e))).astype(np.int64) - 4      # in [0, 4]
    carry = m == 4
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    code_norm = ((e + E5M2_BIAS) << 2) | m

    code = np.where(a < E5M2_MIN_NORMAL, m_sub, code_norm) | sign
    code = np.where(nan, E5M2_NAN, code)
    return code.astype(np.uint8)


def pack_int4(q):
    """Pack 4-bit codes two per byte, element 2j in the low nibble ([FlashComm] Fig. 8
    packs INT4 for transport; the nibble order here is this library's own reading)."""
    q = np.asarray(q, dtype=np.uint8)
    assert q.shape[-1] % 2 == 0
    lo = q[..., 0::2] & 0xF
    hi = q[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(b):
    """Inverse of ``pack_int4``."""
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out
