"""Number-format codecs of the oracle: bf16, fp32, OCP E4M3FN, OCP E2M1, E8M0.

Test infrastructure only (see ``oracle/__init__.py``).

Every routine here works on float64 numpy arrays and is written from the
format definitions, not from any GPU conversion instruction:

* bf16: IEEE-754 binary32 with the low 16 mantissa bits dropped, i.e. 1 sign
  bit, 8 exponent bits (bias 127), 7 mantissa bits, gradual underflow down to
  2^-133; rounding is round-to-nearest, ties-to-even (RN).
* E4M3FN (OCP 8-bit floating point specification, "E4M3" encoding): bias 7,
  3 mantissa bits, no infinities, the only NaN pattern is S.1111.111, largest
  finite magnitude 448 (S.1111.110), subnormals M * 2^-9.
* E2M1 (OCP Microscaling Formats v1.0, FP4 element): bias 1, 1 mantissa bit,
  magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, no NaN/Inf.
* E8M0 (OCP MX v1.0 shared scale): an unsigned biased exponent, value
  2^(byte-127); byte 255 is NaN and is never produced here.

The pages that describe the method fix only the format names (FP8 E4M3 with
FP32 per-128 scales in the Design section of TileScale PR #70; E2M1 weights
sharing one scale per 32 K elements against E4M3 activations in the
Benchmark configuration of FlashInfer PR #6465); the bit-level rules above
come from the OCP documents.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def _round_half_even(v: np.ndarray) -> np.ndarray:
    # numpy's rint rounds halves to the even integer (IEEE roundTiesToEven)
    return np.rint(v)


def _exponent_of_leading_bit(a: np.ndarray) -> np.ndarray:
    """floor(log2(a)) for a > 0, exactly (frexp returns a = m * 2^e, m in [0.5, 1))."""
    _, e = np.frexp(a)
    return e.astype(np.int64) - 1


# ----------------------------------------------------------------------------- bf16 / fp32
def round_fp32(v) -> np.ndarray:
    """RN to IEEE binary32, returned as float64 (numpy's cast is RN-even)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(v) -> np.ndarray:
    """RN (ties to even) of float64 values to bf16, returned as float64.

    One rounding from the exact float64 value (no detour through fp32).
    Overflow beyond the largest finite bf16 gives +-inf.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    with np.errstate(divide="ignore"):
        ebit = np.where(a > 0, _exponent_of_leading_bit(np.where(a > 0, a, 1.0)), -126)
    ebit = np.maximum(ebit, -126)            # below the normal range the quantum stays 2^-133
    q = np.ldexp(1.0, ebit - 7)               # spacing of bf16 values in this binade
    r = _round_half_even(a / q) * q           # a / q is exact: q is a power of two
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(r > bf16_max, np.inf, r)
    return np.copysign(r, v)


def bf16_bits_to_float(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def float_to_bf16_bits(v) -> np.ndarray:
    """float64 values that are exactly representable in bf16 -> uint16 bit patterns."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    if not np.array_equal(f.astype(np.float64), np.asarray(v, dtype=np.float64), equal_nan=True):
        raise ValueError("value not representable in bf16")
    u = f.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("value not representable in bf16")
    return (u >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------- E4M3FN
def e4m3_decode(codes) -> np.ndarray:
    """uint8 E4M3FN codes -> float64 values (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = c & 0x7
    mag = np.where(ex == 0, man * 2.0 ** -9, (1.0 + man / 8.0) * np.ldexp(1.0, ex - 7))
    mag = np.where((ex == 15) & (man == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(u) -> np.ndarray:
    """RN (ties to even) of float64 values to E4M3FN codes, saturating.

    A magnitude that rounds above 448 is replaced by 448 (saturating
    conversion); the sign of zero is kept. Inputs must be finite.
    """
    u = np.asarray(u, dtype=np.float64)
    if not np.all(np.isfinite(u)):
        raise ValueError("e4m3_encode: non-finite input")
    neg = np.signbit(u)
    a = np.abs(u)
    ebit = np.where(a > 0, _exponent_of_leading_bit(np.where(a > 0, a, 1.0)), -6)
    ebit = np.maximum(ebit, -6)               # smallest normal exponent is 1 - 7 = -6
    q = np.ldexp(1.0, ebit - 3)               # 3 mantissa bits
    r = _round_half_even(a / q) * q
    r = np.minimum(r, E4M3_MAX)
    # split the rounded magnitude into exponent and mantissa fields
    er = np.where(r > 0, _exponent_of_leading_bit(np.where(r > 0, r, 1.0)), -7)
    sub = er < -6
    exp_field = np.where(sub, 0, er + 7)
    man_field = np.where(sub, r / 2.0 ** -9, r / np.ldexp(1.0, er - 3) - 8.0)
    code = (exp_field.astype(np.int64) << 3) | man_field.astype(np.int64)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


# ----------------------------------------------------------------------------- E2M1
def e2m1_decode(codes) -> np.ndarray:
    """4-bit E2M1 codes (low nibble of uint8) -> float64 values."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    ex = (c >> 1) & 0x3
    man = c & 0x1
    mag = np.where(ex == 0, man * 0.5, (1.0 + man / 2.0) * np.ldexp(1.0, ex - 1))
    return sign * mag


def e2m1_encode(u) -> np.ndarray:
    """RN (ties to even) of float64 values to E2M1 codes (0..15), saturating at 6."""
    u = np.asarray(u, dtype=np.float64)
    if not np.all(np.isfinite(u)):
        raise ValueError("e2m1_encode: non-finite input")
    neg = np.signbit(u)
    a = np.abs(u)
    ebit = np.where(a > 0, _exponent_of_leading_bit(np.where(a > 0, a, 1.0)), 0)
    ebit = np.maximum(ebit, 0)                # smallest normal exponent is 1 - 1 = 0
    q = np.ldexp(1.0, ebit - 1)               # 1 mantissa bit
    r = _round_half_even(a / q) * q
    r = np.minimum(r, E2M1_MAX)
    er = np.where(r > 0, _exponent_of_leading_bit(np.where(r > 0, r, 1.0)), -1)
    sub = er < 0
    exp_field = np.where(sub, 0, er + 1)
    man_field = np.where(sub, r / 0.5, r / np.ldexp(1.0, er - 1) - 2.0)
    code = (exp_field.astype(np.int64) << 1) | man_field.astype(np.int64)
    code = code | np.where(neg, 0x8, 0)
    return code.astype(np.uint8)


def pack_e2m1(codes) -> np.ndarray:
    """[..., 2n] nibble codes -> [..., n] bytes, even index in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    if c.shape[-1] % 2:
        raise ValueError("pack_e2m1: last dimension must be even")
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_e2m1(packed) -> np.ndarray:
    """[..., n] bytes -> [..., 2n] nibble codes (low nibble first)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ----------------------------------------------------------------------------- E8M0
def e8m0_decode(byte) -> np.ndarray:
    b = np.asarray(byte, dtype=np.uint8).astype(np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))
