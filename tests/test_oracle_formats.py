"""Pins for the oracle's number-format codecs (CPU only).

Each codec is checked against something other than itself: the format
tables of the OCP specifications (tests/golden/), exhaustive nearest-value
search over those tables, torch's library casts, and exact midpoint
constructions.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_bits_to_float(bits)
    return v[np.isfinite(v)]


def _read_table(name):
    vals, rnd = [], []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        parts = line.split()
        if parts[0] == "R":
            rnd.append((float(parts[1]), int(parts[2], 16)))
        else:
            vals.append((int(parts[0], 16), float(parts[1])))
    return vals, rnd


# ------------------------------------------------------------------ bf16 / fp32
def test_round_bf16_matches_torch_on_fp32_inputs():
    # torch's fp32 -> bf16 cast is RN-even; on fp32 inputs there is one rounding
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.0e38)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(F.round_bf16(f.astype(np.float64)), ref)


def test_round_bf16_single_rounding_from_float64():
    # a value just above a bf16 midpoint must round up; double rounding through
    # fp32 would first land on the midpoint and then tie down to even
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert F.round_bf16(v) == 1.0 + 2.0 ** -7
    # exact midpoints tie to the even mantissa
    assert F.round_bf16(1.0 + 2.0 ** -8) == 1.0
    assert F.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2 * 2.0 ** -7
    assert F.round_bf16(-(1.0 + 3 * 2.0 ** -8)) == -(1.0 + 2 * 2.0 ** -7)
    # subnormal spacing 2^-133; sign of zero kept
    assert F.round_bf16(2.0 ** -134) == 0.0
    assert F.round_bf16(2.0 ** -134 + 2.0 ** -140) == 2.0 ** -133
    assert math.copysign(1.0, F.round_bf16(-0.0)) == -1.0


def test_round_bf16_every_midpoint():
    # midpoint between each pair of adjacent positive finite bf16 values
    bits = np.arange(0, 0x7F7F, dtype=np.uint16)
    lo = F.bf16_bits_to_float(bits)
    hi = F.bf16_bits_to_float(bits + 1)
    mid = (lo + hi) / 2                       # exact in float64
    expect = np.where(bits % 2 == 0, lo, hi)  # the even pattern wins
    np.testing.assert_array_equal(F.round_bf16(mid), expect)
    # nudged off the midpoint it goes to the nearer side
    np.testing.assert_array_equal(F.round_bf16(mid + (hi - lo) * 2.0 ** -20), hi)
    np.testing.assert_array_equal(F.round_bf16(mid - (hi - lo) * 2.0 ** -20), lo)


def test_round_fp32_is_ieee():
    assert F.round_fp32(1.0 + 2.0 ** -24) == 1.0
    assert F.round_fp32(1.0 + 2.0 ** -24 + 2.0 ** -40) == 1.0 + 2.0 ** -23


# ------------------------------------------------------------------ E4M3
def test_e4m3_decode_matches_spec_table():
    vals, _ = _read_table("e4m3_spec_values.txt")
    for code, v in vals:
        d = F.e4m3_decode(np.uint8(code))
        if math.isnan(v):
            assert np.isnan(d)
        else:
            assert d == v and math.copysign(1, d) == math.copysign(1, v), hex(code)


def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(F.e4m3_decode(codes), ref)


def _nearest_even(values, table_codes, table_vals):
    """Nearest table value; ties -> the code with mantissa LSB 0."""
    # beyond twice the largest entry the nearest value is the largest entry;
    # capping keeps the float64 distances distinguishable
    values = np.minimum(values, 2 * table_vals.max())
    d = np.abs(values[:, None] - table_vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even = (table_codes[None, :] & 1) == 0
    pick = np.where(cand & even, 1, 0)
    has_even = pick.any(axis=1)
    idx = np.where(has_even, np.argmax(pick, axis=1), np.argmax(cand, axis=1))
    return table_codes[idx]


def test_e4m3_encode_exhaustive_over_bf16():
    v = _all_finite_bf16()
    codes = np.arange(0, 0x7F, dtype=np.int64)          # positive finite codes
    tv = F.e4m3_decode(codes.astype(np.uint8))
    mag = _nearest_even(np.abs(v), codes, tv)          # saturates: 448 is the largest entry
    expect = (mag | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)
    np.testing.assert_array_equal(F.e4m3_encode(v), expect)


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    f = np.concatenate([rng.standard_normal(100000) * 50, rng.standard_normal(50000) * 0.01,
                        np.linspace(-448, 448, 20001)]).astype(np.float32)
    ref = torch.from_numpy(f.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ok = np.abs(f) <= 448
    np.testing.assert_array_equal(F.e4m3_encode(f[ok].astype(np.float64)), ref[ok])


def test_e4m3_saturation_and_midpoints():
    assert F.e4m3_encode(464.0) == 0x7E       # tie between 448 (even) and 480 -> 448
    assert F.e4m3_encode(470.0) == 0x7E       # would round to 480: saturates
    assert F.e4m3_encode(-1e30) == 0xFE
    assert F.e4m3_encode(2.0 ** -10) == 0x00  # half the min subnormal: tie to even 0
    assert F.e4m3_encode(3 * 2.0 ** -10) == 0x02
    assert F.e4m3_encode(-0.0) == 0x80


# ------------------------------------------------------------------ E2M1
def test_e2m1_tables():
    vals, rnd = _read_table("e2m1_spec_values.txt")
    for code, v in vals:
        d = F.e2m1_decode(np.uint8(code))
        assert d == v and math.copysign(1, d) == math.copysign(1, v), hex(code)
    for v, code in rnd:
        assert F.e2m1_encode(v) == code, v


def test_e2m1_encode_exhaustive_over_bf16():
    v = _all_finite_bf16()
    codes = np.arange(0, 8, dtype=np.int64)
    tv = F.e2m1_decode(codes.astype(np.uint8))
    mag = _nearest_even(np.abs(v), codes, tv)
    expect = (mag | np.where(np.signbit(v), 0x8, 0)).astype(np.uint8)
    np.testing.assert_array_equal(F.e2m1_encode(v), expect)


def test_e2m1_pack_order():
    codes = np.array([[0x1, 0x2, 0xF, 0x7]], dtype=np.uint8)
    packed = F.pack_e2m1(codes)
    assert packed.tolist() == [[0x21, 0x7F]]       # even index in the low nibble
    np.testing.assert_array_equal(F.unpack_e2m1(packed), codes)


def test_e8m0_decode():
    assert F.e8m0_decode(np.uint8(127)) == 1.0
    assert F.e8m0_decode(np.uint8(0)) == 2.0 ** -127
    assert F.e8m0_decode(np.uint8(254)) == 2.0 ** 127
    assert np.isnan(F.e8m0_decode(np.uint8(255)))


@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan])
def test_encoders_reject_non_finite(bad):
    with pytest.raises(ValueError):
        F.e4m3_encode(np.array([bad]))
    with pytest.raises(ValueError):
        F.e2m1_encode(np.array([bad]))
