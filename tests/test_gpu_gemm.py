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
from tests.gpu_util import U32, assert_within_rounding, cuda, f64, say

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
