"""GPU parity of route, align_sort, the quantisers and combine against the
oracle, through the C ABI (bit-exact for integer / code outputs)."""
import numpy as np
import pytest
import torch

import mixture_experts_routed_top_amd as M
from oracle import formats as F
from oracle import moe as O
from workloads import get_config, make_inputs
from tests.gpu_util import U32, assert_route_weights, assert_within_rounding, cuda, f64, say

pytestmark = pytest.mark.gpu


def _bf16_tensor(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)


# ------------------------------------------------------------------ route
ROUTE_CASES = [
    ("tiny_bf16", None), ("qwen3_30b_a3b_bf16", None), ("qwen3_30b_a3b_bf16_zipf", None),
    ("llama4_scout_bf16", None), ("mxfp4_moe_t1024", None), ("fp8_block128_share", 257),
]


@pytest.mark.parametrize("name,T", ROUTE_CASES)
def test_route_matches_oracle(name, T):
    cfg = get_config(name)
    if T is not None:
        cfg = cfg.with_(T=T)
    inp = make_inputs(cfg, with_weights=False)
    say("route", name, cfg.T, cfg.E, cfg.k)
    ids, w = M.moe_route(cuda(inp.logits), cfg.k, cfg.score)
    torch.cuda.synchronize()
    rid, rw = O.route(inp.logits.numpy(), cfg.k, cfg.score)
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    assert_route_weights(w.cpu().numpy(), rw)


@pytest.mark.parametrize("T,E,k,score", [(1, 1, 1, 0), (7, 3, 3, 0), (33, 1024, 32, 0), (5, 64, 1, 1),
                                         (300, 65, 7, 0), (100, 16, 4, 1)])
def test_route_edges_and_ties(T, E, k, score):
    rng = np.random.default_rng(T * E + k)
    logits = rng.integers(-2, 3, size=(T, E)).astype(np.float32)   # many exact ties
    logits[0, :] = 0.0
    if E > 1:
        logits[-1, 1] = -0.0
    say("route-ties", T, E, k, score)
    ids, w = M.moe_route(cuda(torch.from_numpy(logits)), k, score)
    torch.cuda.synchronize()
    rid, rw = O.route(logits, k, score)
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    assert_route_weights(w.cpu().numpy(), rw)


def _candidate_logits(T, E, k, kind, rng):
    if kind == "normal":
        return rng.standard_normal((T, E)).astype(np.float32)
    if kind == "top_ties":                      # the largest logit repeated on a few experts
        x = rng.standard_normal((T, E)).astype(np.float32)
        for t in range(T):
            x[t, rng.choice(E, size=min(E, k + 3), replace=False)] = x[t].max()
        return x
    if kind == "ints":                          # many exact ties everywhere
        return rng.integers(-50, 51, size=(T, E)).astype(np.float32)
    # k = 1 and the maximum on exactly 64 (row 0) or 65 (row 1) experts, the
    # most and one more than the candidate select takes; the rest below it
    x = rng.uniform(-1.0, 0.5, size=(T, E)).astype(np.float32)
    for t in range(T):
        x[t, rng.choice(E, size=64 + (t % 2), replace=False)] = 3.0
    return x


@pytest.mark.parametrize("T,E,k,kind", [(300, 129, 5, "normal"), (300, 200, 16, "top_ties"), (257, 256, 8, "ints"),
                                        (300, 300, 1, "normal"), (300, 512, 10, "top_ties"),
                                        (200, 512, 32, "normal"), (300, 1000, 20, "ints"),
                                        (4, 512, 1, "max_64_65"), (4, 1024, 1, "max_64_65")])
def test_route_candidate_select(T, E, k, kind):
    """More than 128 experts: the select over the keys at or above the k-th
    largest lane maximum (at most 64 of them), or over every key when more
    are; ids and weights as the oracle, ties to the lower expert."""
    rng = np.random.default_rng(T * E + k)
    logits = _candidate_logits(T, E, k, kind, rng)
    say("route-candidates", T, E, k, kind)
    ids, w = M.moe_route(cuda(torch.from_numpy(logits)), k, O.SCORE_SOFTMAX)
    torch.cuda.synchronize()
    rid, rw = O.route(logits, k, O.SCORE_SOFTMAX)
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    assert_route_weights(w.cpu().numpy(), rw)


@pytest.mark.parametrize("T,E,k,S", [(100, 16, 4, 1), (33, 64, 8, 3), (5, 4, 2, 2), (257, 512, 10, 1)])
def test_route_shared_matches_oracle(T, E, k, S):
    rng = np.random.default_rng(T + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    say("route-shared", T, E, k, S)
    ids, w = M.moe_route_shared(cuda(torch.from_numpy(logits)), k, O.SCORE_SOFTMAX, S)
    torch.cuda.synchronize()
    rid, rw = O.route_with_shared(logits, k, O.SCORE_SOFTMAX, S)
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    assert_route_weights(w.cpu().numpy(), rw)
    assert np.all(w.cpu().numpy()[:, k:] == 1.0)


# ------------------------------------------------------------------ align_sort
def _align_check(ids_np, E, bm, runs=1):
    T, k = ids_np.shape
    say("align_sort", T, k, E, bm)
    ids = cuda(torch.from_numpy(ids_np.astype(np.int32)))
    outs = []
    for _ in range(runs):
        s = M.moe_align_sort(ids, E, bm)
        torch.cuda.synchronize()
        outs.append(s)
    counts, offsets, sorted_ids, tile_expert, num_tiles = O.align_sort(ids_np, E, bm)
    for s in outs:
        np.testing.assert_array_equal(s.counts.cpu().numpy(), counts)
        np.testing.assert_array_equal(s.offsets.cpu().numpy(), offsets)
        np.testing.assert_array_equal(s.sorted_ids.cpu().numpy()[:len(sorted_ids)], sorted_ids)
        np.testing.assert_array_equal(s.tile_expert.cpu().numpy()[:len(tile_expert)], tile_expert)
        assert int(s.num_tiles.item()) == num_tiles


@pytest.mark.parametrize("bm", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("name", ["tiny_bf16", "qwen3_30b_a3b_bf16", "qwen3_30b_a3b_bf16_zipf",
                                  "mxfp4_moe_t16384", "llama4_scout_bf16"])
def test_align_sort_matches_oracle(name, bm):
    cfg = get_config(name)
    inp = make_inputs(cfg, with_weights=False)
    ids, _ = O.route(inp.logits.numpy(), cfg.k, cfg.score)
    _align_check(ids, cfg.E, bm, runs=2)


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (511, 4, 2), (512, 4, 2), (513, 4, 2), (1023, 1, 1),
                                   (1025, 3, 1), (40, 1024, 7), (3000, 512, 10),
                                   # at 16384 assignments and just past it
                                   (2048, 128, 8), (2049, 128, 8), (16384, 1024, 1), (16385, 7, 1),
                                   # at 2048 assignments (the one-workgroup sort) and just past it
                                   (256, 64, 8), (257, 64, 8), (2048, 1024, 1), (683, 3, 3)])
def test_align_sort_edges(T, E, k):
    rng = np.random.default_rng(T + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _align_check(ids, E, 16)
    _align_check(ids, E, 256)


# Problems with more than 2048 (expert, chunk) counts take the one-launch
# scan-and-scatter whose 1024 threads split the experts into 1024 // E slices:
# one slice (E = 1000), E not dividing 1024 (E = 7, 146 slices), one expert
# over 2051 chunks (1024 slices, two chunks each), and a ragged last chunk.
@pytest.mark.parametrize("T,E,k", [(3000, 1000, 1), (300000, 7, 1), (2100000, 1, 1), (8191, 256, 3)])
def test_align_sort_wide_scan(T, E, k):
    rng = np.random.default_rng(T * 7 + E)
    if k == 1:
        ids = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    else:
        ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    _align_check(ids, E, 32)
    _align_check(ids, E, 256)


def test_align_sort_all_tokens_one_expert():
    ids = np.full((2048, 1), 3, np.int32)        # experts 0..2 and 4..7 empty
    _align_check(ids, 8, 64)


# ------------------------------------------------------------------ quantisers
def _finite_bf16_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_bits_to_float(bits)
    return v[np.isfinite(v)]


def _blocks_with_anchor(values, block, anchor):
    """Rows of `block` values, the last of each row = anchor (fixes the block scale)."""
    per = block - 1
    n = -(-len(values) // per)
    pad = np.zeros(n * per - len(values))
    body = np.concatenate([values, pad]).reshape(n, per)
    return np.concatenate([body, np.full((n, 1), anchor)], axis=1)


def test_fp8_encoder_exhaustive_over_bf16():
    # every finite bf16 value in a 1x128 block whose amax is 448 (scale 1); the
    # values beyond 448 take the saturating path, so clip them into [-448, 448]
    v = _finite_bf16_patterns()
    v = v[np.abs(v) <= 448]
    blocks = _blocks_with_anchor(v, 128, 448.0)
    x = cuda(_bf16_tensor(blocks))
    say("fp8 exhaustive", blocks.shape)
    q, s = M.moe_quantize_fp8(x, 1)
    torch.cuda.synchronize()
    rq, rs = O.quantize_fp8_block(blocks, 1, 128)
    assert np.all(rs == 1.0)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


@pytest.mark.parametrize("rows,cols,br,std", [(64, 7168, 1, 1.0), (3, 128, 1, 1e-3), (256, 384, 128, 0.02),
                                               (128, 2048, 128, 3.0)])
def test_fp8_block_quant_matches_oracle(rows, cols, br, std):
    rng = np.random.default_rng(rows + cols)
    v = f64(_bf16_tensor(rng.standard_normal((rows, cols)) * std))
    v[0, :128] = 0.0                                  # an all-zero block
    say("fp8 quant", rows, cols, br)
    q, s = M.moe_quantize_fp8(cuda(_bf16_tensor(v)), br)
    torch.cuda.synchronize()
    rq, rs = O.quantize_fp8_block(v, br, 128)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


def test_mxfp8_encoder_exhaustive_over_bf16():
    v = _finite_bf16_patterns()
    v = v[np.abs(v) < 300]
    blocks = _blocks_with_anchor(v, 32, 300.0)                    # amax in [256, 512): X = 1
    say("mxfp8 exhaustive", blocks.shape)
    q, sb = M.moe_quantize_mxfp8(cuda(_bf16_tensor(blocks)))
    torch.cuda.synchronize()
    rq, rsb = O.quantize_mxfp8(blocks)
    np.testing.assert_array_equal(sb.cpu().numpy(), rsb)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


def test_mxfp4_encoder_exhaustive_over_bf16():
    v = _finite_bf16_patterns()
    v = v[np.abs(v) < 7]
    blocks = _blocks_with_anchor(v, 32, 7.0)                      # amax in [4, 8): X = 1
    say("mxfp4 exhaustive", blocks.shape)
    q, sb = M.moe_quantize_mxfp4(cuda(_bf16_tensor(blocks)))
    torch.cuda.synchronize()
    rq, rsb = O.quantize_mxfp4(blocks)
    np.testing.assert_array_equal(sb.cpu().numpy(), rsb)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


@pytest.mark.parametrize("rows,cols,std", [(64, 2560, 1.0), (1280, 640, 0.02), (5, 64, 1e-30)])
def test_mx_quant_random_matches_oracle(rows, cols, std):
    rng = np.random.default_rng(cols)
    v = f64(_bf16_tensor(rng.standard_normal((rows, cols)) * std))
    v[1, 32:64] = 0.0
    x = cuda(_bf16_tensor(v))
    say("mx quant", rows, cols, std)
    q8, s8 = M.moe_quantize_mxfp8(x)
    q4, s4 = M.moe_quantize_mxfp4(x)
    torch.cuda.synchronize()
    r8, rs8 = O.quantize_mxfp8(v)
    r4, rs4 = O.quantize_mxfp4(v)
    np.testing.assert_array_equal(s8.cpu().numpy(), rs8)
    np.testing.assert_array_equal(q8.cpu().numpy(), r8)
    np.testing.assert_array_equal(s4.cpu().numpy(), rs4)
    np.testing.assert_array_equal(q4.cpu().numpy(), r4)


# ------------------------------------------------------------------ combine
@pytest.mark.parametrize("T,k,H", [(129, 8, 2048), (1, 1, 8), (64, 2, 256), (37, 10, 2560), (3, 32, 7168),
                                   # every slot count from 3 to 9 (the kernel is specialised for k <= 10)
                                   (17, 3, 1024), (17, 4, 1024), (19, 5, 512), (50, 6, 2688), (11, 7, 256),
                                   (21, 9, 2048)])
def test_combine_matches_oracle(T, k, H):
    rng = np.random.default_rng(T * k)
    y = f64(_bf16_tensor(rng.standard_normal((T * k, H))))
    w = rng.random((T, k)).astype(np.float32)
    w /= w.sum(1, keepdims=True)
    say("combine", T, k, H)
    out = M.moe_combine(cuda(_bf16_tensor(y)), cuda(torch.from_numpy(w)))
    torch.cuda.synchronize()
    ref = O.combine(y, w)
    got = f64(out)
    # k fp32 fused multiply-adds in slot order versus a float64 sum: the fp32
    # sum is within k * 2^-24 * sum_j |w_j y_j| of the exact one
    delta = k * U32 * np.abs(w.astype(np.float64)[:, :, None] * y.reshape(T, k, H)).sum(1)
    assert_within_rounding(got, ref, delta, min_exact=0.98)
    if k == 1:
        np.testing.assert_array_equal(got, np.where(w[:, :1] == 1.0, y, got))
