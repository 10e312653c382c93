"""Pins for the oracle's quantisers (CPU only).

The FP8 block quantiser is compared with an independent torch implementation
that does the same fp32 arithmetic (torch's IEEE fp32 division and its
float8_e4m3fn cast); the MX quantisers with a torch / table implementation of
the OCP MX v1.0 conversion; plus round-trip error bounds and the property
that the largest element of a block lands on the top of the code range.
"""
import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import moe as O


def _bf16_values(shape, std, seed):
    rng = np.random.default_rng(seed)
    v = (rng.standard_normal(shape) * std).astype(np.float32)
    return torch.from_numpy(v).to(torch.bfloat16).float().numpy().astype(np.float64)


def _torch_fp8_block(v, br, bc):
    t = torch.from_numpy(v.astype(np.float32))
    R, C = t.shape
    b = t.reshape(R // br, br, C // bc, bc)
    amax = b.abs().amax(dim=(1, 3))
    s = amax / torch.tensor(448.0, dtype=torch.float32)
    s = torch.where(amax == 0, torch.ones_like(s), s)
    q = (b / s[:, None, :, None]).clamp(-448, 448)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(R, C)
    return codes.numpy(), s.numpy()


@pytest.mark.parametrize("br", [1, 128])
def test_fp8_block_matches_torch(br):
    v = _bf16_values((256, 384), 0.5, br)
    v[0:br, 128:256] = 0.0                     # an all-zero block: scale 1, codes 0
    codes, s = O.quantize_fp8_block(v, br, 128)
    rc, rs = _torch_fp8_block(v, br, 128)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(codes, rc)
    assert s[0, 1] == 1.0


def test_fp8_block_round_trip_bound_and_max_code():
    v = _bf16_values((64, 1024), 3.0, 11)
    codes, s = O.quantize_fp8_block(v, 1, 128)
    deq = O.dequantize_fp8_block(codes, s, 1, 128)
    sb = np.repeat(s.astype(np.float64), 128, axis=1)
    normal = np.abs(v) / sb >= 2.0 ** -6
    # 3 mantissa bits: half an ulp is 2^-4 of the leading bit
    assert np.all(np.abs(deq - v)[normal] <= 2.0 ** -4 * np.abs(v)[normal] * (1 + 2 ** -20))
    assert np.all(np.abs(deq - v)[~normal] <= 2.0 ** -10 * sb[~normal] * (1 + 2 ** -20))
    # the block maximum maps to +-448 (code 0x7E / 0xFE)
    mag = codes & 0x7F
    assert np.all(mag.reshape(64, 8, 128).max(axis=2) == 0x7E)


def _torch_mx_scale(v, emax):
    t = torch.from_numpy(v.reshape(v.shape[0], -1, 32))
    amax = t.abs().amax(dim=-1)
    _, e = torch.frexp(amax)
    x = torch.clamp(e.to(torch.int64) - 1 - emax, -127, 127)
    x = torch.where(amax == 0, torch.full_like(x, -127), x)
    return (x + 127).to(torch.uint8).numpy()


def test_mxfp8_matches_torch():
    v = _bf16_values((64, 256), 2.0, 5)
    v[3, 32:64] = 0.0
    codes, sb = O.quantize_mxfp8(v)
    rsb = _torch_mx_scale(v, 8)
    np.testing.assert_array_equal(sb, rsb)
    x = np.ldexp(1.0, rsb.astype(np.int64) - 127)
    q = torch.from_numpy((v.reshape(64, -1, 32) / x[..., None]).astype(np.float32)).clamp(-448, 448)
    rc = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(64, 256).numpy()
    np.testing.assert_array_equal(codes, rc)
    assert sb[3, 1] == 0
    # largest element: amax / X lies in [256, 512) -> code magnitude in [256, 448]
    deq_mag = np.abs(F.e4m3_decode(codes)).reshape(64, -1, 32).max(-1)
    nz = sb != 0
    assert np.all((deq_mag[nz] >= 256) & (deq_mag[nz] <= 448))


def test_mxfp4_matches_table_nearest():
    v = _bf16_values((32, 512), 0.02, 9)
    packed, sb = O.quantize_mxfp4(v)
    rsb = _torch_mx_scale(v, 2)
    np.testing.assert_array_equal(sb, rsb)
    x = np.repeat(np.ldexp(1.0, rsb.astype(np.int64) - 127), 32, axis=1)
    u = v / x
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    a = np.minimum(np.abs(u), 12.0)
    d = np.abs(a[..., None] - grid)
    best = d.min(-1, keepdims=True)
    cand = d == best
    even = (np.arange(8) & 1) == 0
    idx = np.where((cand & even).any(-1), np.argmax(cand & even, -1), np.argmax(cand, -1))
    ref = (idx | np.where(np.signbit(u), 8, 0)).astype(np.uint8)
    np.testing.assert_array_equal(F.unpack_e2m1(packed), ref)
    # largest element of each block: amax / X in [4, 8) -> code magnitude 4 or 6
    mags = np.abs(F.e2m1_decode(F.unpack_e2m1(packed))).reshape(32, -1, 32).max(-1)
    assert np.all((mags == 4) | (mags == 6))


def test_mx_shared_exponent_clamps():
    v = np.zeros((1, 64))
    v[0, :32] = 2.0 ** -130                    # tiny block: exponent clamps to -127
    v[0, 32] = 2.0 ** 130                      # huge block (not bf16 range, rule only)
    _, sb = O.quantize_mxfp8(v)
    assert sb[0, 0] == 0 and sb[0, 1] == 127 + 122


def test_quantisers_reject_ragged_shapes():
    with pytest.raises(ValueError):
        O.quantize_fp8_block(np.zeros((3, 100)), 1, 128)
    with pytest.raises(ValueError):
        O.quantize_mxfp8(np.zeros((3, 40)))
    with pytest.raises(ValueError):
        O.quantize_mxfp4(np.zeros((3, 40)))
