"""GPU parity of the grouped GEMMs (GEMM1 + SwiGLU, GEMM2) against the oracle.

The sorted layout fed to the kernels comes from the oracle, so these tests do
not depend on the GPU align_sort. Integer-valued operands make every fp32
accumulation exact, which pins the GEMMs bit for bit; random operands are
checked against the rounding bound of fp32 accumulation (n * 2^-24 * sum of
|terms|) plus one bf16 step, and must agree exactly on >= 99% of elements."""
import numpy as np
import pytest
import torch

import mixture_experts_routed_top_amd as M
from oracle import moe as O
from tests.gpu_util import F8F6F4_GROUP_LOSS, U32, assert_within_rounding, cuda, f64, say

pytestmark = pytest.mark.gpu


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)


def _sort_from_oracle(ids, E, bm):
    T, k = ids.shape
    s = M.SortResult(T, k, E, bm, "cuda:0")
    counts, offsets, sorted_ids, tile_expert, num_tiles = O.align_sort(ids, E, bm)
    s.counts.copy_(torch.from_numpy(counts))
    s.offsets.copy_(torch.from_numpy(offsets))
    s.sorted_ids[:len(sorted_ids)].copy_(torch.from_numpy(sorted_ids))
    s.tile_expert[:len(tile_expert)].copy_(torch.from_numpy(tile_expert))
    s.num_tiles.fill_(num_tiles)
    return s, (sorted_ids, tile_expert, num_tiles)


def _gate_up(xs, w1, sorted_ids, tile_expert, num_tiles, bm, k, rows):
    """Per sorted row: (x_row @ W1[e, :I].T, x_row @ W1[e, I:].T) for operands xs, w1."""
    I = w1.shape[1] // 2
    A = xs.shape[0] * k
    g = np.zeros((rows, I))
    u = np.zeros((rows, I))
    for t in range(num_tiles):
        e = tile_expert[t]
        a = sorted_ids[t * bm:(t + 1) * bm].astype(np.int64)
        ok = a < A
        xa = np.zeros((bm, xs.shape[1]))
        xa[ok] = xs[a[ok] // k]
        g[t * bm:(t + 1) * bm] = xa @ w1[e, :I].T
        u[t * bm:(t + 1) * bm] = xa @ w1[e, I:].T
    return g, u


def _abs_sums(x, w1, *a):
    return _gate_up(np.abs(x), np.abs(w1), *a)


def _values(x, w1, *a):
    return _gate_up(x, w1, *a)


def _problem(T, H, E, k, I, seed, integer):
    rng = np.random.default_rng(seed)
    if integer:
        x = rng.integers(-2, 3, (T, H)).astype(np.float64)
        w1 = rng.integers(-2, 3, (E, 2 * I, H)).astype(np.float64)
        w2 = rng.integers(-2, 3, (E, H, I)).astype(np.float64)
    else:
        x = f64(_bf16(rng.standard_normal((T, H))))
        w1 = f64(_bf16(rng.standard_normal((E, 2 * I, H)) * 0.05))
        w2 = f64(_bf16(rng.standard_normal((E, H, I)) * 0.05))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = O.route(logits, k)
    return x, w1, w2, ids


SHAPES = [  # T, H, E, k, I, block_m
    (64, 256, 8, 2, 128, 32),      # the tiny BF16 workload
    (64, 192, 4, 2, 96, 32),       # partial tiles on every GEMM edge
    (129, 384, 16, 4, 256, 64),    # hidden divisible by 8 but not by 256; ragged T
    (1, 256, 8, 2, 128, 32),
    (300, 2048, 128, 8, 768, 128), # the Qwen3-30B-A3B expert shape at small T
    (200, 200, 8, 3, 40, 64),      # K tails of one 8-column chunk
    (700, 2048, 8, 4, 768, 256),   # 256-row tiles: several full tiles per expert, ragged last tiles
    (300, 384, 16, 4, 136, 256),   # 256-row tiles with partial column tiles and a K tail
    # 256-row tiles run a six-step pipeline loop: k-step counts 1, 4 / 2, 5 / 7, 1
    # (GEMM1 K = H, GEMM2 K = I; 64 K a step) end it at every position
    (260, 64, 4, 2, 200, 256),
    (300, 120, 4, 2, 312, 256),
    (280, 448, 4, 2, 64, 256),
    # 256-row tiles, I % 256 == 64: the squared-ReLU GEMM1 covers the last
    # 64 columns with a second launch of 128-column tiles
    (300, 640, 8, 4, 320, 256),
]


@pytest.mark.parametrize("integer", [True, False])
@pytest.mark.parametrize("T,H,E,k,I,bm", SHAPES)
def test_gemm1_swiglu_bf16(T, H, E, k, I, bm, integer):
    x, w1, w2, ids = _problem(T, H, E, k, I, T + H + I, integer)
    sort, (sorted_ids, tile_expert, num_tiles) = _sort_from_oracle(ids, E, bm)
    say("gemm1 bf16", T, H, E, k, I, bm, integer)
    h, _ = M.moe_grouped_gemm_swiglu(M.DTYPE_BF16, cuda(_bf16(x)), None, cuda(_bf16(w1)), None, sort, H, I)
    torch.cuda.synchronize()
    rows = num_tiles * bm
    (ref, _), _ = O.grouped_gemm_swiglu(x, w1, sorted_ids, tile_expert, num_tiles, bm, k, O.DTYPE_BF16)
    got = f64(h[:rows])
    # fp32 accumulation of H products: |g' - g| <= H 2^-24 sum|x w| (same for u);
    # silu' is at most 1.1 in magnitude, and expf / the division add a few ulps
    ga, ua = _abs_sums(x, w1, sorted_ids, tile_expert, num_tiles, bm, k, rows)
    gv, uv = _values(x, w1, sorted_ids, tile_expert, num_tiles, bm, k, rows)
    sig = 1.0 / (1.0 + np.exp(-np.clip(gv, -700, 700)))
    silu = gv * sig
    dg, du = H * U32 * ga, H * U32 * ua
    delta = 1.1 * dg * (np.abs(uv) + du) + np.abs(silu) * du + 8 * U32 * np.abs(silu * uv)
    # integer operands: g*u often lands exactly on a bf16 midpoint in fp32
    # (silu(g) == g in fp32 for large g) while the exact value sits just below
    # it, so ties legitimately break the other way more often than for random data
    assert_within_rounding(got, ref, delta, min_exact=0.97 if integer else 0.99)
    pad = sorted_ids[:rows] == T * k
    assert np.all(got[pad] == 0)


@pytest.mark.parametrize("integer", [True, False])
@pytest.mark.parametrize("T,H,E,k,I,bm", SHAPES)
def test_gemm1_relu2_bf16(T, H, E, k, I, bm, integer):
    """The ungated squared-ReLU GEMM1 (W1 [E, I, H])."""
    x, w1g, _, ids = _problem(T, H, E, k, I, T + 3 * H + I, integer)
    w1 = np.ascontiguousarray(w1g[:, :I])
    sort, (sorted_ids, tile_expert, num_tiles) = _sort_from_oracle(ids, E, bm)
    say("gemm1 relu2 bf16", T, H, E, k, I, bm, integer)
    h, _ = M.moe_grouped_gemm_relu2(M.DTYPE_BF16, cuda(_bf16(x)), None, cuda(_bf16(w1)), None, sort, H, I)
    torch.cuda.synchronize()
    rows = num_tiles * bm
    (ref, _), _ = O.grouped_gemm_swiglu(x, w1, sorted_ids, tile_expert, num_tiles, bm, k, O.DTYPE_BF16,
                                        act=O.ACT_RELU2)
    got = f64(h[:rows])
    # g: fp32 accumulation of H products, |g' - g| <= dg = H 2^-24 sum|x w|;
    # h = max(g, 0)^2 then moves by at most (2|g| + dg) dg, plus one fp32
    # rounding of the square
    w_both = np.concatenate([w1, w1], axis=1)
    ga, _ = _abs_sums(x, w_both, sorted_ids, tile_expert, num_tiles, bm, k, rows)
    gv, _ = _values(x, w_both, sorted_ids, tile_expert, num_tiles, bm, k, rows)
    dg = H * U32 * ga
    delta = (2 * np.abs(gv) + dg) * dg + 2 * U32 * gv * gv
    assert_within_rounding(got, ref, delta, min_exact=0.99)
    assert np.all(got >= 0)
    pad = sorted_ids[:rows] == T * k
    assert np.all(got[pad] == 0)


@pytest.mark.parametrize("integer", [True, False])
@pytest.mark.parametrize("T,H,E,k,I,bm", SHAPES)
def test_gemm2_down_bf16(T, H, E, k, I, bm, integer):
    x, w1, w2, ids = _problem(T, H, E, k, I, T + 7 * H + I, integer)
    sort, (sorted_ids, tile_expert, num_tiles) = _sort_from_oracle(ids, E, bm)
    rows = num_tiles * bm
    rng = np.random.default_rng(5)
    hval = (rng.integers(-3, 4, (sort.cap, I)).astype(np.float64) if integer
            else f64(_bf16(rng.standard_normal((sort.cap, I)))))
    say("gemm2 bf16", T, H, E, k, I, bm, integer)
    y = torch.full((T * k, H), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    M.moe_grouped_gemm_down(M.DTYPE_BF16, cuda(_bf16(hval)), None, cuda(_bf16(w2)), None, sort, H, I, y=y)
    torch.cuda.synchronize()
    ref = O.grouped_gemm_down(hval[:rows], w2, sorted_ids, tile_expert, num_tiles, bm, T * k)
    got = f64(y)
    assert not np.isnan(got).any()          # every assignment row written
    if integer:
        np.testing.assert_array_equal(got, ref)
    else:
        absref = O.grouped_gemm_down(np.abs(hval[:rows]), np.abs(w2), sorted_ids, tile_expert, num_tiles, bm,
                                     T * k)
        assert_within_rounding(got, ref, 1.01 * I * U32 * absref, min_exact=0.99)


def test_gemm_bitwise_invariant_to_block_m_layout():
    # the same assignments laid out with different paddings give the same Y
    T, H, E, k, I = 100, 256, 8, 2, 128
    x, w1, w2, ids = _problem(T, H, E, k, I, 77, False)
    ys = []
    for bm in (32, 64, 128):
        sort, _ = _sort_from_oracle(ids, E, bm)
        say("gemm layout invariance", bm)
        h, _ = M.moe_grouped_gemm_swiglu(M.DTYPE_BF16, cuda(_bf16(x)), None, cuda(_bf16(w1)), None, sort, H, I)
        y = M.moe_grouped_gemm_down(M.DTYPE_BF16, h, None, cuda(_bf16(w2)), None, sort, H, I)
        torch.cuda.synchronize()
        ys.append(y.cpu())
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[0], ys[2])


# ============================================================ FP8 128-block and MX paths
def _fp8_operands(x, w1, w2, integer):
    """Oracle-quantised operands (codes, scales) for the FP8 path.

    integer: small-integer values encoded exactly with unit scales, so every
    product and every fp32 partial sum is exact."""
    from oracle import formats as F
    E, twoI, H = w1.shape
    I = twoI // 2
    if integer:
        xq, xs = F.e4m3_encode(x), np.ones((x.shape[0], H // 128), np.float32)
        w1q, w1s = F.e4m3_encode(w1.reshape(E * twoI, H)), np.ones((E * twoI // 128, H // 128), np.float32)
        w2q, w2s = F.e4m3_encode(w2.reshape(E * H, I)), np.ones((E * H // 128, I // 128), np.float32)
    else:
        xq, xs = O.quantize_fp8_block(x, 1, 128)
        w1q, w1s = O.quantize_fp8_block(w1.reshape(E * twoI, H), 128, 128)
        w2q, w2s = O.quantize_fp8_block(w2.reshape(E * H, I), 128, 128)
    deq = (O.dequantize_fp8_block(xq, xs, 1, 128),
           O.dequantize_fp8_block(w1q, w1s, 128, 128).reshape(w1.shape),
           O.dequantize_fp8_block(w2q, w2s, 128, 128).reshape(w2.shape))
    return (xq, xs), (w1q, w1s), (w2q, w2s), deq


def _mx_operands(x, w1, w2, integer):
    from oracle import formats as F
    E, twoI, H = w1.shape
    I = twoI // 2
    if integer:
        xq, xs = F.e4m3_encode(x), np.full((x.shape[0], H // 32), 127, np.uint8)
        w1q = F.pack_e2m1(F.e2m1_encode(w1.reshape(E * twoI, H)))
        w1s = np.full((E * twoI, H // 32), 127, np.uint8)
        w2q = F.pack_e2m1(F.e2m1_encode(w2.reshape(E * H, I)))
        w2s = np.full((E * H, I // 32), 127, np.uint8)
    else:
        xq, xs = O.quantize_mxfp8(x)
        w1q, w1s = O.quantize_mxfp4(w1.reshape(E * twoI, H))
        w2q, w2s = O.quantize_mxfp4(w2.reshape(E * H, I))
    deq = (O.dequantize_mxfp8(xq, xs), O.dequantize_mxfp4(w1q, w1s).reshape(w1.shape),
           O.dequantize_mxfp4(w2q, w2s).reshape(w2.shape))
    return (xq, xs), (w1q, w1s), (w2q, w2s), deq


def _t(a):
    return cuda(torch.from_numpy(np.ascontiguousarray(a)))


SCALED_SHAPES = [  # T, H, E, k, I, block_m
    (64, 256, 8, 2, 128, 32),
    (129, 384, 16, 4, 256, 64),
    (300, 1024, 32, 8, 512, 128),
    (1, 256, 4, 2, 128, 32),
    (700, 1024, 8, 4, 384, 256),   # 256-row tiles: full and ragged tiles, partial column tiles
    (200, 640, 8, 2, 384, 32),     # 32-row tiles with an odd number of 128-K steps in both GEMMs
    # 128-row tiles with I % 256 == 128: the MX GEMM1 takes the last 128 columns in a second launch
    (300, 512, 8, 4, 384, 128),
    (257, 1024, 16, 4, 640, 128),
    # 64- to 256-row tiles split their LDS stages and run a six-step pipeline
    # loop: with the shapes above, k-step counts 7 and 1 (H = 896, I = 128)
    # end it at every position
    (150, 896, 4, 2, 128, 64),
    (600, 896, 4, 2, 128, 256),
]


def _int_problem(T, H, E, k, I, seed, dtype):
    rng = np.random.default_rng(seed)
    vals = np.array([-3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3]) if dtype == M.DTYPE_MXFP4W_MXFP8A \
        else np.arange(-4, 5).astype(np.float64)
    x = rng.integers(-3, 4, (T, H)).astype(np.float64)
    w1 = rng.choice(vals, (E, 2 * I, H))
    w2 = rng.choice(vals, (E, H, I))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = O.route(logits, k)
    return x, w1, w2, ids


@pytest.mark.parametrize("dtype", [M.DTYPE_FP8_BLOCK128, M.DTYPE_MXFP4W_MXFP8A])
@pytest.mark.parametrize("integer", [True, False])
@pytest.mark.parametrize("T,H,E,k,I,bm", SCALED_SHAPES)
def test_gemm2_down_scaled(T, H, E, k, I, bm, integer, dtype):
    if integer:
        x, w1, w2, ids = _int_problem(T, H, E, k, I, T + H, dtype)
    else:
        x, w1, w2, ids = _problem(T, H, E, k, I, T + 3 * H + I, False)
    sort, (sorted_ids, tile_expert, num_tiles) = _sort_from_oracle(ids, E, bm)
    rows = num_tiles * bm
    rng = np.random.default_rng(11)
    # h operand: codes and scales straight from the oracle's quantiser of a random h
    hraw = rng.integers(-4, 5, (sort.cap, I)).astype(np.float64) if integer else \
        f64(_bf16(rng.standard_normal((sort.cap, I))))
    ops = _fp8_operands if dtype == M.DTYPE_FP8_BLOCK128 else _mx_operands
    _, _, (w2q, w2s), (_, _, w2h) = ops(x, w1, w2, integer)
    if dtype == M.DTYPE_FP8_BLOCK128:
        from oracle import formats as F
        hq, hs = (F.e4m3_encode(hraw), np.ones((sort.cap, I // 128), np.float32)) if integer else \
            O.quantize_fp8_block(hraw, 1, 128)
        hhat = O.dequantize_fp8_block(hq, hs, 1, 128)
    else:
        from oracle import formats as F
        hq, hs = (F.e4m3_encode(hraw), np.full((sort.cap, I // 32), 127, np.uint8)) if integer else \
            O.quantize_mxfp8(hraw)
        hhat = O.dequantize_mxfp8(hq, hs)
    say("gemm2 scaled", dtype, T, H, E, k, I, bm, integer)
    y = torch.full((T * k, H), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    M.moe_grouped_gemm_down(dtype, _t(hq), _t(hs), _t(w2q), _t(w2s), sort, H, I, y=y)
    torch.cuda.synchronize()
    ref = O.grouped_gemm_down(hhat[:rows], w2h, sorted_ids, tile_expert, num_tiles, bm, T * k)
    got = f64(y)
    assert not np.isnan(got).any()
    if integer:
        np.testing.assert_array_equal(got, ref)
    else:
        absref = O.grouped_gemm_down(np.abs(hhat[:rows]), np.abs(w2h), sorted_ids, tile_expert, num_tiles, bm,
                                     T * k)
        # fp32 accumulation, plus (FP8) the promotion's roundings per 128-group, plus
        # what the f8f6f4 MFMA drops when it aligns each group of 8 products
        assert_within_rounding(got, ref, (1.05 * (I + 3 * I // 128) * U32 + 1.01 * F8F6F4_GROUP_LOSS) * absref,
                               min_exact=0.98)


def _check_h_quant(dtype, hq_gpu, hs_gpu, href, rows, I, delta):
    """Requantised h from the kernel versus the float64 h of the same operands.

    delta bounds |h_fp32 - h| elementwise (fp32 accumulation in the kernel)."""
    from oracle import formats as F
    hq_gpu, hs_gpu = hq_gpu[:rows], hs_gpu[:rows]
    if dtype == M.DTYPE_FP8_BLOCK128:
        deq = O.dequantize_fp8_block(hq_gpu, hs_gpu, 1, 128)
        # every non-zero 1x128 block has its maximum on the top code (+-448)
        mag = (hq_gpu & 0x7F).reshape(rows, I // 128, 128).max(-1)
        nz = np.abs(href).reshape(rows, I // 128, 128).max(-1) > 0
        assert np.all(mag[nz] == 0x7E)
        scale = np.repeat(hs_gpu.astype(np.float64), 128, axis=1)
    else:
        deq = O.dequantize_mxfp8(hq_gpu, hs_gpu)
        mag = np.abs(F.e4m3_decode(hq_gpu)).reshape(rows, I // 32, 32).max(-1)
        nz = hs_gpu != 0
        assert np.all((mag[nz] >= 256) & (mag[nz] <= 448))
        scale = np.repeat(F.e8m0_decode(hs_gpu), 32, axis=1)
    # E4M3 rounding: half an ulp is 2^-4 of |v| for normal codes and 2^-10 of
    # the scale for subnormal ones, applied to the kernel's fp32 h (within
    # delta of h). MX blocks may clip: magnitudes above 448 X become 448 X.
    target = np.clip(href, -448 * scale, 448 * scale)
    lim = (1.01 / 16) * (np.abs(target) + delta) + delta + scale / 512 + 1e-30
    bad = np.abs(deq - target) > lim
    if bad.any():
        r, c = np.argwhere(bad)[0]
        blk = 128 if dtype == M.DTYPE_FP8_BLOCK128 else 32
        b0 = (c // blk) * blk
        raise AssertionError(f"{bad.sum()} of {bad.size} elements off; first at row {r} col {c}: h={href[r, c]:.6g} "
                             f"deq={deq[r, c]:.6g} scale={scale[r, c]:.6g} block amax(h)="
                             f"{np.abs(href[r, b0:b0 + blk]).max():.6g} code={hq_gpu[r, c]:#x}")
    return deq


@pytest.mark.parametrize("dtype", [M.DTYPE_FP8_BLOCK128, M.DTYPE_MXFP4W_MXFP8A])
@pytest.mark.parametrize("T,H,E,k,I,bm", SCALED_SHAPES)
def test_gemm1_swiglu_scaled(T, H, E, k, I, bm, dtype):
    x, w1, w2, ids = _problem(T, H, E, k, I, T + 5 * H + I, False)
    sort, (sorted_ids, tile_expert, num_tiles) = _sort_from_oracle(ids, E, bm)
    rows = num_tiles * bm
    ops = _fp8_operands if dtype == M.DTYPE_FP8_BLOCK128 else _mx_operands
    (xq, xs), (w1q, w1s), _, (xh, w1h, _) = ops(x, w1, w2, False)
    say("gemm1 scaled", dtype, T, H, E, k, I, bm)
    hq, hs = M.moe_grouped_gemm_swiglu(dtype, _t(xq), _t(xs), _t(w1q), _t(w1s), sort, H, I)
    torch.cuda.synchronize()
    # float64 h from the same dequantised operands, before its storage point
    g, u = _values(xh, w1h, sorted_ids, tile_expert, num_tiles, bm, k, rows)
    sig = 1.0 / (1.0 + np.exp(-np.clip(g, -700, 700)))
    href = g * sig * u
    # fp32 accumulation of H products, plus (FP8) the promotion's roundings
    # per 128-group, plus the f8f6f4 MFMA's group alignment, for g and for u
    ga, ua = _abs_sums(xh, w1h, sorted_ids, tile_expert, num_tiles, bm, k, rows)
    eps = (H + 3 * H // 128) * U32 + F8F6F4_GROUP_LOSS
    dg, du = eps * ga, eps * ua
    delta = 1.1 * dg * (np.abs(u) + du) + np.abs(g * sig) * du + 8 * U32 * np.abs(href)
    deq = _check_h_quant(dtype, hq.cpu().numpy(), hs.cpu().numpy(), href, rows, I, delta)
    (ref_codes, _ref_scales), ref_val = O.grouped_gemm_swiglu(xh, w1h, sorted_ids, tile_expert, num_tiles, bm, k,
                                                              dtype)
    assert np.linalg.norm(deq - ref_val) <= 0.02 * np.linalg.norm(ref_val) + 1e-30
    # codes agree with the oracle's requantisation of its own float64 h except
    # where the fp32 and float64 h straddle a rounding boundary
    assert np.mean(hq.cpu().numpy()[:rows] == ref_codes) > 0.97


# Shapes whose weight walk exceeds 4 MB, so the FP8 / MX kernels take the
# grouped task order with 32-, 64- and 128-row tiles (GEMM1: 2 I H = 4.7 MB
# per m-tile walk; GEMM2: H I = 4.7 MB), several m-tiles per expert.
GROUPED_SCALED_SHAPES = [(400, 2048, 4, 2, 2304, bm) for bm in (32, 64, 128)]


@pytest.mark.parametrize("dtype", [M.DTYPE_FP8_BLOCK128, M.DTYPE_MXFP4W_MXFP8A])
@pytest.mark.parametrize("T,H,E,k,I,bm", GROUPED_SCALED_SHAPES)
def test_gemm1_swiglu_scaled_grouped_order(T, H, E, k, I, bm, dtype):
    test_gemm1_swiglu_scaled(T, H, E, k, I, bm, dtype)


@pytest.mark.parametrize("dtype", [M.DTYPE_FP8_BLOCK128, M.DTYPE_MXFP4W_MXFP8A])
@pytest.mark.parametrize("T,H,E,k,I,bm", GROUPED_SCALED_SHAPES)
def test_gemm2_down_scaled_grouped_order(T, H, E, k, I, bm, dtype):
    test_gemm2_down_scaled(T, H, E, k, I, bm, False, dtype)


# ------------------------------------------------------------ storage rounding of h, bit for bit
CANARY = 0x5A


def _canary_like(shape, dtype):
    """A tensor of `shape` followed by a band of 8 canary rows, every byte CANARY."""
    t = torch.empty((shape[0] + 8,) + tuple(shape[1:]), dtype=dtype, device="cuda:0")
    t.view(torch.uint8).fill_(CANARY)
    return t


def _untouched(t, first_row):
    """Every byte of rows first_row.. still holds the canary."""
    return bool((t[first_row:].contiguous().view(torch.uint8) == CANARY).all().item())


H32_SHAPES = {  # dtype -> shapes (T, H, E, k, I, block_m)
    M.DTYPE_BF16: [SHAPES[0], SHAPES[1], SHAPES[2], SHAPES[6], SHAPES[7]],
    M.DTYPE_FP8_BLOCK128: SCALED_SHAPES + GROUPED_SCALED_SHAPES[:1],
    M.DTYPE_MXFP4W_MXFP8A: SCALED_SHAPES + GROUPED_SCALED_SHAPES[:1],
}


@pytest.mark.parametrize("dtype,T,H,E,k,I,bm", [(d,) + s for d, ss in H32_SHAPES.items() for s in ss])
def test_gemm1_storage_rounding_bitexact(dtype, T, H, E, k, I, bm):
    """The kernel's own fp32 h (moe_grouped_gemm_swiglu_h32), fed through the
    oracle's storage rounding, gives the kernel's stored h bit for bit: bf16
    RN, or FP8 1x128 codes and fp32 scales, or MXFP8 1x32 codes and E8M0
    scales. The h32 variant stores exactly what the plain call stores; rows
    past num_tiles * block_m and the canary rows after cap stay untouched;
    h32 is within the fp32 accumulation bound of the float64 h."""
    from oracle import formats as F
    x, w1, w2, ids = _problem(T, H, E, k, I, T + 9 * H + I, False)
    sort, (sorted_ids, tile_expert, num_tiles) = _sort_from_oracle(ids, E, bm)
    rows, cap = num_tiles * bm, sort.cap
    if dtype == M.DTYPE_BF16:
        xa, xs, w1a, w1s = cuda(_bf16(x)), None, cuda(_bf16(w1)), None
        xh, w1h = x, w1
        hdt, sdt, sg = torch.bfloat16, None, 1
    else:
        ops = _fp8_operands if dtype == M.DTYPE_FP8_BLOCK128 else _mx_operands
        (xq, xsc), (w1q, w1sc), _, (xh, w1h, _) = ops(x, w1, w2, False)
        xa, xs, w1a, w1s = _t(xq), _t(xsc), _t(w1q), _t(w1sc)
        hdt = torch.uint8
        sdt, sg = (torch.float32, 128) if dtype == M.DTYPE_FP8_BLOCK128 else (torch.uint8, 32)
    say("gemm1 storage rounding", dtype, T, H, E, k, I, bm)
    h = _canary_like((cap, I), hdt)
    hs = _canary_like((cap, I // sg), sdt) if sdt is not None else None
    h32 = _canary_like((cap, I), torch.float32)
    M.moe_grouped_gemm_swiglu_h32(dtype, xa, xs, w1a, w1s, sort, H, I, h[:cap], None if hs is None else hs[:cap],
                                  h32[:cap])
    hp, hsp = M.moe_grouped_gemm_swiglu(dtype, xa, xs, w1a, w1s, sort, H, I)
    torch.cuda.synchronize()
    # the h32 variant writes what the plain call writes
    assert torch.equal(h[:rows].view(torch.uint8), hp[:rows].view(torch.uint8))
    if hs is not None:
        assert torch.equal(hs[:rows].view(torch.uint8), hsp[:rows].view(torch.uint8))
    # untouched: rows past num_tiles * block_m and the canary band after cap
    assert _untouched(h, rows) and _untouched(h32, rows)
    assert hs is None or _untouched(hs, rows)
    v32 = h32[:rows].cpu().numpy().astype(np.float64)
    # storage rounding of the kernel's own fp32 h: bit for bit
    if dtype == M.DTYPE_BF16:
        np.testing.assert_array_equal(f64(h[:rows]), F.round_bf16(v32))
    elif dtype == M.DTYPE_FP8_BLOCK128:
        qref, sref = O.quantize_fp8_block(v32, 1, 128)
        np.testing.assert_array_equal(h[:rows].cpu().numpy(), qref)
        np.testing.assert_array_equal(hs[:rows].cpu().numpy().view(np.uint32), sref.view(np.uint32))
    else:
        qref, sref = O.quantize_mxfp8(v32)
        np.testing.assert_array_equal(h[:rows].cpu().numpy(), qref)
        np.testing.assert_array_equal(hs[:rows].cpu().numpy(), sref)
    # the fp32 h itself: within the accumulation bound of the float64 h of the same operands
    g, u = _values(xh, w1h, sorted_ids, tile_expert, num_tiles, bm, k, rows)
    sig = 1.0 / (1.0 + np.exp(-np.clip(g, -700, 700)))
    href = g * sig * u
    ga, ua = _abs_sums(xh, w1h, sorted_ids, tile_expert, num_tiles, bm, k, rows)
    eps = H * U32 if dtype == M.DTYPE_BF16 else (H + 3 * H // 128) * U32 + F8F6F4_GROUP_LOSS
    dg, du = eps * ga, eps * ua
    delta = 1.1 * dg * (np.abs(u) + du) + np.abs(g * sig) * du + 8 * U32 * np.abs(href)
    bad = np.abs(v32 - href) > delta + 1e-37
    assert not bad.any(), f"{bad.sum()} fp32 h values beyond the accumulation bound"
    pad = sorted_ids[:rows] == T * k
    assert np.all(v32[pad] == 0)


# ------------------------------------------------------------ FP8 per-128 promotion: dynamic range
@pytest.mark.parametrize("bm", [32, 128, 256])
def test_fp8_promotion_tiny_and_huge_blocks(bm):
    """Tokens whose 1x128 blocks differ hugely in magnitude (one block scaled
    by 2^-110, another by 2^+40, so block scales span about 2^150) and
    weight blocks scaled by 2^-40: the per-128 promotion must stay finite
    and match the float64 GEMMs of the same dequantised operands, in GEMM1
    and in GEMM2 (h scales of some blocks cut by 2^-100)."""
    T, H, E, k, I = 96, 512, 4, 2, 256
    rng = np.random.default_rng(123)
    x = f64(_bf16(rng.standard_normal((T, H))))
    x[::3, 0:128] *= 2.0 ** -110          # tiny first block in every third token
    x[1::3, 256:384] *= 2.0 ** 40         # huge third block in others
    w1 = f64(_bf16(rng.standard_normal((E, 2 * I, H)) * 0.05))
    w1[:, :, 384:512] *= 2.0 ** -40       # a tiny K block of every weight row
    w2 = f64(_bf16(rng.standard_normal((E, H, I)) * 0.05))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = O.route(logits, k)
    sort, (sorted_ids, tile_expert, num_tiles) = _sort_from_oracle(ids, E, bm)
    rows = num_tiles * bm
    (xq, xs), (w1q, w1s), (w2q, w2s), (xh, w1h, w2h) = _fp8_operands(x, w1, w2, False)
    say("fp8 promotion range", bm)
    hq, hs, h32 = M.moe_grouped_gemm_swiglu_h32(M.DTYPE_FP8_BLOCK128, _t(xq), _t(xs), _t(w1q), _t(w1s), sort, H, I)
    torch.cuda.synchronize()
    v32 = h32[:rows].cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(v32))
    g, u = _values(xh, w1h, sorted_ids, tile_expert, num_tiles, bm, k, rows)
    href = g / (1.0 + np.exp(-np.clip(g, -700, 700))) * u
    ga, ua = _abs_sums(xh, w1h, sorted_ids, tile_expert, num_tiles, bm, k, rows)
    eps = (H + 3 * H // 128) * U32 + F8F6F4_GROUP_LOSS
    dg, du = eps * ga, eps * ua
    sig = 1.0 / (1.0 + np.exp(-np.clip(g, -700, 700)))
    delta = 1.1 * dg * (np.abs(u) + du) + np.abs(g * sig) * du + 8 * U32 * np.abs(href)
    assert not (np.abs(v32 - href) > delta + 1e-37).any()
    qref, sref = O.quantize_fp8_block(v32, 1, 128)
    np.testing.assert_array_equal(hq[:rows].cpu().numpy(), qref)
    np.testing.assert_array_equal(hs[:rows].cpu().numpy().view(np.uint32), sref.view(np.uint32))
    # GEMM2 on the same h codes, with h scales spanning a wide range too
    hs_np = hs[:sort.cap].cpu().numpy().copy()
    hs_np[: rows: 5, 0] *= np.float32(2.0 ** -100)
    hhat = O.dequantize_fp8_block(hq[:sort.cap].cpu().numpy(), hs_np, 1, 128)
    y = torch.full((T * k, H), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    M.moe_grouped_gemm_down(M.DTYPE_FP8_BLOCK128, hq, _t(hs_np), _t(w2q), _t(w2s), sort, H, I, y=y)
    torch.cuda.synchronize()
    got = f64(y)
    assert np.all(np.isfinite(got))
    ref = O.grouped_gemm_down(hhat[:rows], w2h, sorted_ids, tile_expert, num_tiles, bm, T * k)
    absref = O.grouped_gemm_down(np.abs(hhat[:rows]), np.abs(w2h), sorted_ids, tile_expert, num_tiles, bm, T * k)
    assert_within_rounding(got, ref, (1.05 * (I + 3 * I // 128) * U32 + 1.01 * F8F6F4_GROUP_LOSS) * absref,
                           min_exact=0.98)


# ------------------------------------------------------------ K-split of a short last round (BF16)
WS_COUNTER_BYTES = 8192   # the grouped-GEMM workspace starts with its counters (split slots, queues)
SPLIT_SHAPES = [  # T, H, E, k, I; round-robin routing: 640 rows per expert, 3 tiles of 256 each (48 tiles)
    (2560, 512, 16, 4, 1024),    # GEMM1 (K = 512): 384 tasks, a last round of 16 per XCD of 32 workgroups
    (2560, 2048, 16, 4, 512),    # GEMM2 (K = 512): 384 tasks, likewise
]


@pytest.mark.parametrize("T,H,E,k,I", SPLIT_SHAPES)
def test_bf16_gemms_k_split_last_round(T, H, E, k, I):
    """Given the workspace, the BF16 GEMMs cut the tiles of a short last round
    in two along K and add the two fp32 halves. h and Y stay within the fp32
    accumulation bound of the float64 oracle; h is still RN_bf16 of the
    kernel's own fp32 h, bit for bit; a second call is bitwise identical; the
    workspace's counters are zero again after every call; and on a 256-CU GPU, where these
    shapes leave a last round of 16 tiles per XCD, the split tiles' fp32 sums
    differ from the unsplit call's somewhere (the split ran)."""
    from oracle import formats as F
    bm = 256
    rng = np.random.default_rng(T + H + I)
    x = f64(_bf16(rng.standard_normal((T, H))))
    w1 = f64(_bf16(rng.standard_normal((E, 2 * I, H)) * 0.05))
    w2 = f64(_bf16(rng.standard_normal((E, H, I)) * 0.05))
    ids = (np.arange(T * k) % E).reshape(T, k).astype(np.int32)
    sort, (sorted_ids, tile_expert, num_tiles) = _sort_from_oracle(ids, E, bm)
    rows = num_tiles * bm
    assert num_tiles == 48
    say("bf16 k-split", T, H, E, k, I)
    ws = M.moe_grouped_gemm_workspace("cuda:0")
    xa, w1a, w2a = cuda(_bf16(x)), cuda(_bf16(w1)), cuda(_bf16(w2))
    h0, _, h32_0 = M.moe_grouped_gemm_swiglu_h32(M.DTYPE_BF16, xa, None, w1a, None, sort, H, I)
    h1, _, h32_1 = M.moe_grouped_gemm_swiglu_h32(M.DTYPE_BF16, xa, None, w1a, None, sort, H, I, ws=ws)
    torch.cuda.synchronize()
    assert not ws[:WS_COUNTER_BYTES].any()     # the counters; the rest holds partial tiles
    h2, _ = M.moe_grouped_gemm_swiglu(M.DTYPE_BF16, xa, None, w1a, None, sort, H, I, ws=ws)
    y0 = M.moe_grouped_gemm_down(M.DTYPE_BF16, h1, None, w2a, None, sort, H, I)
    y1 = M.moe_grouped_gemm_down(M.DTYPE_BF16, h1, None, w2a, None, sort, H, I, ws=ws)
    y2 = M.moe_grouped_gemm_down(M.DTYPE_BF16, h1, None, w2a, None, sort, H, I, ws=ws)
    torch.cuda.synchronize()
    assert not ws[:WS_COUNTER_BYTES].any()     # the counters; the rest holds partial tiles
    assert torch.equal(h1[:rows], h2[:rows]) and torch.equal(y1, y2)
    v32 = h32_1[:rows].cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(f64(h1[:rows]), F.round_bf16(v32))
    # h: the fp32 h within the accumulation bound of the float64 h (a split sum has fewer rounding steps
    # on any path than the H-term sequential one)
    g, u = _values(x, w1, sorted_ids, tile_expert, num_tiles, bm, k, rows)
    sig = 1.0 / (1.0 + np.exp(-np.clip(g, -700, 700)))
    href = g * sig * u
    ga, ua = _abs_sums(x, w1, sorted_ids, tile_expert, num_tiles, bm, k, rows)
    dg, du = H * U32 * ga, H * U32 * ua
    delta = 1.1 * dg * (np.abs(u) + du) + np.abs(g * sig) * du + 8 * U32 * np.abs(href)
    assert not (np.abs(v32 - href) > delta + 1e-37).any()
    # Y from the kernel's own h
    hval = f64(h1[:rows])
    yref = O.grouped_gemm_down(hval, w2, sorted_ids, tile_expert, num_tiles, bm, T * k)
    yabs = O.grouped_gemm_down(np.abs(hval), np.abs(w2), sorted_ids, tile_expert, num_tiles, bm, T * k)
    assert_within_rounding(f64(y1), yref, 1.01 * I * U32 * yabs, min_exact=0.99)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        split_ran = not torch.equal(h32_0[:rows], h32_1[:rows]) if H == 512 else not torch.equal(y0, y1)
        assert split_ran, "the last round was not split"
