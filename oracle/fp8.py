"""OCP FP8 E4M3FN codec and bf16 helpers, written from the format definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Format (OCP 8-bit floating point, E4M3 "fn" variant), the byte encoding the
cache stores. The pages name it three ways: torch's ``float8_e4m3fn`` dtype
(FlashMLA PR #82 "update fp8 support", the H800 test report), "OCP e4m3", the
encoding gfx950 reads (ROCm/aiter PR #6199, Technical details), and the
amax/448 quantization rule, 448 being the format's largest finite value
(InfiniCore PR #1568, Summary, FP8 KV cache bullet).

  bit 7      sign
  bits 6..3  exponent E, bias 7
  bits 2..0  mantissa M
  E == 0           subnormal: (M/8) * 2**-6
  E in 1..15       normal:    (1 + M/8) * 2**(E-7)
  E == 15, M == 7  NaN (0x7F and 0xFF); there is no infinity
so the largest finite magnitude is 0x7E = 1.75 * 2**8 = 448 and the smallest
subnormal is 2**-9.

Pinned by tests/test_oracle_fp8.py: anchor codes, a second derivation by bf16
bit placement (InfiniCore PR #1568, mma kernel commit: placing the code bits in
bf16 bit positions gives the true value times 2**-120), encode/decode round
trip, round-half-to-even ties, saturation, and torch's float8_e4m3fn cast as an
outside library check. The e4m3fnuz decoder below is pinned the same way:
torch's float8_e4m3fnuz on all 256 codes, the page's largest value 240, its
special codes, and the bias identity with e4m3fn on the other 253 codes.
"""

import math

import numpy as np

E4M3FN_MAX = 448.0


def _e4m3fn_value(code: int) -> float:
    """Value of one e4m3fn byte, straight from the bit-field definition."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


#: float64 value of every byte 0..255 (NaN at 0x7F and 0xFF).
E4M3FN_TABLE = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)
E4M3FN_TABLE.setflags(write=False)

# Non-negative finite codes 0x00..0x7E are strictly increasing in value, so
# "nearest code" is a search over this sorted list.
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = E4M3FN_TABLE[:0x7F].copy()


def decode_e4m3fn(codes) -> np.ndarray:
    """Bytes -> float64 values (table lookup)."""
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        c = c.astype(np.uint8)
    return E4M3FN_TABLE[c]


# ---- e4m3fnuz (gfx942) -------------------------------------------------------
# The one-byte float of gfx942 that ROCm/aiter PR #6199 (Technical details)
# quantizes to, saturating at 240. Its bit fields, from the format's
# definition:
#   bit 7 sign, bits 6..3 exponent E with bias 8, bits 2..0 mantissa M
#   E == 0           subnormal: (M/8) * 2**-7
#   E in 1..15       normal:    (1 + M/8) * 2**(E-8)   (no NaN among them)
#   0x80             NaN (the "negative zero" code); 0x00 is the only zero
# so the largest magnitude is 0x7F = 1.875 * 2**7 = 240 and the smallest
# subnormal is 2**-10.

E4M3FNUZ_MAX = 240.0


def _e4m3fnuz_value(code: int) -> float:
    """Value of one e4m3fnuz byte, straight from the bit-field definition."""
    if code == 0x80:
        return math.nan
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -7
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 8)


#: float64 value of every byte 0..255 (NaN at 0x80 only).
E4M3FNUZ_TABLE = np.array([_e4m3fnuz_value(c) for c in range(256)], dtype=np.float64)
E4M3FNUZ_TABLE.setflags(write=False)


def decode_e4m3fnuz(codes) -> np.ndarray:
    """Bytes -> float64 values of the e4m3fnuz encoding (table lookup)."""
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        c = c.astype(np.uint8)
    return E4M3FNUZ_TABLE[c]


def decode_kv_codes(codes, encoding="e4m3fn") -> np.ndarray:
    """Cache code bytes -> float64 under the named one-byte encoding."""
    if encoding == "e4m3fn":
        return decode_e4m3fn(codes)
    if encoding == "e4m3fnuz":
        return decode_e4m3fnuz(codes)
    raise ValueError(f"unknown encoding {encoding!r}")


def fnuz_as_e4m3fn(codes) -> np.ndarray:
    """e4m3fnuz bytes -> the e4m3fn bytes of the same values, for fp8 matrix
    cores that read OCP codes only (ROCm/aiter PR #6199, Technical details:
    gfx942's fnuz against gfx950's OCP e4m3).

    Each fnuz value is encoded as e4m3fn by round to nearest, ties to even
    (``encode_e4m3fn``). Every fnuz magnitude from 2**-6 up to 240 is an
    e4m3fn value (e4m3fn reaches 448), so those codes keep their value
    exactly; below 2**-6 fnuz steps by 2**-10 and e4m3fn by 2**-9, so half of
    those 15 magnitudes round. 0x80, fnuz's NaN, is taken as zero (-0, 0x80),
    as the decode reads it.
    """
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        c = c.astype(np.uint8)
    v = decode_e4m3fnuz(c)
    v = np.where(c == 0x80, -0.0, v)
    return encode_e4m3fn(v)


def encode_e4m3fn(x) -> np.ndarray:
    """float64 -> e4m3fn bytes: round to nearest, ties to even, saturating.

    Magnitudes at or above 448 map to 0x7E (saturation); NaN maps to 0x7F.
    Ties between two neighbouring codes go to the code whose mantissa LSB is
    0, which is the even code number because codes are monotone in value.
    """
    v = np.asarray(x, dtype=np.float64)
    mag = np.abs(v)
    mag_c = np.minimum(mag, E4M3FN_MAX)
    hi = np.searchsorted(_POS_VALUES, mag_c, side="left")  # first value >= mag
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    v_hi = _POS_VALUES[hi]
    v_lo = _POS_VALUES[lo]
    d_hi = v_hi - mag_c
    d_lo = mag_c - v_lo
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    pick_hi |= (hi == lo)
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    # The sign is kept, as in IEEE rounding: a negative value that rounds to
    # zero gives -0 (0x80).
    code = np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)
    code = np.where(np.isnan(v), np.uint8(0x7F), code).astype(np.uint8)
    return code


def e4m3fn_by_bf16_bit_placement(codes) -> np.ndarray:
    """Second derivation of the decode, independent of the bit-field formula.

    The 7 exponent+mantissa bits are placed at bf16 bit positions 10..4 and the
    sign at bit 15. Read as bf16 this equals the true value times 2**-120
    (bf16 has 7 mantissa bits and exponent bias 127 = 7 + 120), for normals and
    subnormals alike. Valid for finite codes only.
    """
    c = np.asarray(codes).astype(np.uint32)
    bits = ((c & 0x80) << 8) | ((c & 0x7F) << 4)
    return bf16_bits_to_f64(bits.astype(np.uint16)) * 2.0 ** 120


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    b = np.asarray(bits).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even.

    NaN maps to the quiet NaN 0x7FC0 (sign kept).
    """
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    r = np.where(nan, (((u >> 16) & 0x8000) | 0x7FC0).astype(np.uint16), r)
    return r.astype(np.uint16)
