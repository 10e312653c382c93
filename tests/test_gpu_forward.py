"""End-to-end GPU forward (route -> align_sort -> GEMM1+SwiGLU -> GEMM2 ->
combine, all through the C ABI) against the oracle.

Small problems are compared on every output element; the full-size
workloads, in the launch configuration the benchmark times, are compared on
all routing / layout outputs and on a sample of tokens that the oracle
evaluates one by one."""
import os

import numpy as np
import pytest
import torch

import mixture_experts_routed_top_amd as M
from oracle import moe as O
from workloads import P5_GRID, get_config, make_inputs, make_inputs_device, to_f64
from tests.gpu_util import (TOL_COS, TOL_FRO, U32, assert_route_weights, assert_within_rounding, cuda, f64,
                            min_row_cos, rel_fro, say)

pytestmark = pytest.mark.gpu


def _run(cfg, inp, block_m=None):
    layer = M.MoeLayer(cfg.dtype, cuda(inp.w1), cuda(inp.w2), cfg.k, cfg.score, cfg.act, cfg.n_shared)
    plan = layer.plan(cfg.T, block_m=block_m)
    out = layer(cuda(inp.x), cuda(inp.logits), plan)
    torch.cuda.synchronize()
    return layer, plan, out


def _full_compare(cfg, inp, block_m=None):
    say("forward full", cfg.name, cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, block_m)
    layer, plan, out = _run(cfg, inp, block_m)
    ref = O.moe_forward(inp.logits.numpy(), to_f64(inp.x), to_f64(inp.w1), to_f64(inp.w2), cfg.k, cfg.score,
                        cfg.dtype, block_m=plan.block_m, act=cfg.act, n_shared=cfg.n_shared)
    np.testing.assert_array_equal(plan.ids.cpu().numpy(), ref["ids"])
    np.testing.assert_array_equal(plan.sort.sorted_ids.cpu().numpy()[:len(ref["sorted_ids"])], ref["sorted_ids"])
    got = f64(out)
    assert rel_fro(got, ref["out"]) <= TOL_FRO[cfg.dtype]
    assert min_row_cos(got, ref["out"]) >= TOL_COS
    return got, ref


def test_tiny_bf16_forward():
    cfg = get_config("tiny_bf16")
    got, ref = _full_compare(cfg, make_inputs(cfg))
    assert rel_fro(got, ref["out"]) < 4e-3


@pytest.mark.parametrize("T,H,E,k,I", [(1, 256, 8, 2, 128), (7, 256, 8, 2, 128), (129, 384, 16, 4, 256),
                                       (64, 192, 4, 2, 96), (8191 // 16, 2048, 128, 8, 768),
                                       (100, 1024, 1, 1, 512)])
def test_bf16_forward_edge_shapes(T, H, E, k, I):
    cfg = get_config("tiny_bf16").with_(T=T, H=H, E=E, k=k, I=I, w_std=0.05)
    _full_compare(cfg, make_inputs(cfg, seed=T))


def test_bf16_forward_grouped_m_tiles():
    """256-row tiles (GEMM1: 16 n-tiles of 256 rows x 2048; GEMM2: 8 n-tiles
    of 256 rows x 2048); the tasks walk the n-tiles with each expert's m-tiles
    side by side in both GEMMs, and 5 experts with one m-tile each make groups
    of one."""
    cfg = get_config("tiny_bf16").with_(T=700, H=2048, E=5, k=1, I=2048, w_std=0.02)
    _full_compare(cfg, make_inputs(cfg, seed=21), block_m=256)


def test_bf16_forward_expert_groups_long_runs():
    """Each expert's m-tiles walk the n-tiles in groups of up to four (GEMM1:
    16 n-tiles of 256 rows x 1536; GEMM2: 6 n-tiles of 256 rows x 2048, above
    the 4 MB walk the FP8 / MX kernels group from too); one expert holds 37
    m-tiles (runs of more than 32 tiles on both sides of most of its tiles,
    and a last group of one), the others 3 and 2. Routing and layout are
    compared in full, Y on rows from every m-tile."""
    cfg = get_config("tiny_bf16").with_(T=10300, H=1536, E=3, k=1, I=2048, w_std=0.02)
    inp = make_inputs(cfg, seed=5)
    inp.logits[:] = -1.0
    inp.logits[:9300, 0] = 2.0
    inp.logits[9300:10000, 1] = 2.0
    inp.logits[10000:, 2] = 2.0
    say("forward expert groups", cfg.T, cfg.H, cfg.E, cfg.I)
    layer, plan, out = _run(cfg, inp, block_m=256)
    rid, rw = O.route_with_shared(inp.logits.numpy(), cfg.k, cfg.score, 0)
    np.testing.assert_array_equal(plan.ids.cpu().numpy(), rid)
    counts, offsets, sorted_ids, tile_expert, num_tiles = O.align_sort(rid, cfg.E, 256)
    assert list(np.bincount(tile_expert[:num_tiles], minlength=3)) == [37, 3, 2]
    np.testing.assert_array_equal(plan.sort.sorted_ids.cpu().numpy()[:len(sorted_ids)], sorted_ids)
    np.testing.assert_array_equal(plan.sort.tile_expert.cpu().numpy()[:len(tile_expert)], tile_expert)
    rng = np.random.default_rng(1)
    assigned, refs = [], []
    for e in range(cfg.E):
        seg = sorted_ids[offsets[e]:offsets[e] + counts[e]]
        # the first and last row of every 256-row tile, and one more in each
        pick = np.unique(np.concatenate([seg[0::256], seg[255::256], [seg[-1]],
                                         seg[np.minimum(np.arange(0, len(seg), 256) + 97, len(seg) - 1)]]))
        w1e, w2e = to_f64(inp.w1[e]), to_f64(inp.w2[e])
        xr = to_f64(inp.x[torch.from_numpy(pick)])
        refs += [O.assignment_forward(xr[i], w1e, w2e, cfg.dtype, cfg.act) for i in range(len(pick))]
        assigned += list(pick)
    got = f64(plan.y[torch.from_numpy(np.array(assigned)).to(out.device)])
    ref = np.stack(refs)
    assert rel_fro(got, ref) <= TOL_FRO[cfg.dtype]
    assert min_row_cos(got, ref) >= TOL_COS
    assert torch.isfinite(out.float()).all()


def test_bf16_forward_expert_groups_very_long_run():
    """One expert with 117 m-tiles of 256 rows: the 64-tile continuation of the
    grouped order's expert-run search takes several rounds in both
    directions; small H and I keep the full oracle comparison cheap."""
    cfg = get_config("tiny_bf16").with_(T=30000, H=64, E=2, k=1, I=64, w_std=0.05)
    inp = make_inputs(cfg, seed=6)
    inp.logits[:] = -1.0
    inp.logits[:29900, 0] = 2.0
    inp.logits[29900:, 1] = 2.0
    _full_compare(cfg, inp, block_m=256)


def test_bf16_forward_one_expert_takes_all():
    cfg = get_config("tiny_bf16").with_(T=300, E=8, k=1)
    inp = make_inputs(cfg, seed=3)
    inp.logits[:] = -1.0
    inp.logits[:, 5] = 2.0        # every token -> expert 5; the others stay empty
    _full_compare(cfg, inp)


def test_bf16_forward_deterministic():
    cfg = get_config("tiny_bf16").with_(T=513, E=16, k=4)
    inp = make_inputs(cfg, seed=9)
    say("forward determinism")
    _, _, a = _run(cfg, inp)
    _, _, b = _run(cfg, inp)
    assert torch.equal(a, b)


_WCACHE = {}


def _inputs_cached(cfg):
    """Inputs of a full-size workload; the expert weights are generated once
    per weight shape (the token-count sweep of one workload shares them)."""
    key = (cfg.cfg_id, cfg.E, cfg.H, cfg.I, cfg.w_std)
    if key not in _WCACHE:
        _WCACHE.clear()
        full = make_inputs(cfg)
        _WCACHE[key] = (full.w1, full.w2)
    inp = make_inputs(cfg, with_weights=False)
    inp.w1, inp.w2 = _WCACHE[key]
    return inp


def _oracle_expert(cfg, layer, e, w1e, w2e):
    """The oracle's quantisation of expert e, dequantised; for the FP8 / MX
    paths the GPU's own weight codes for e must equal the oracle's bit for bit."""
    if cfg.dtype == O.DTYPE_BF16:
        return w1e, w2e
    twoI, H = 2 * cfg.I, cfg.H
    if cfg.dtype == O.DTYPE_FP8_BLOCK128:
        (q1, s1), (q2, s2) = O.quantize_fp8_block(w1e, 128, 128), O.quantize_fp8_block(w2e, 128, 128)
        np.testing.assert_array_equal(layer.w1_scale[e * twoI // 128:(e + 1) * twoI // 128].cpu().numpy(), s1)
        np.testing.assert_array_equal(layer.w2_scale[e * H // 128:(e + 1) * H // 128].cpu().numpy(), s2)
        d1, d2 = O.dequantize_fp8_block(q1, s1, 128, 128), O.dequantize_fp8_block(q2, s2, 128, 128)
    else:
        (q1, s1), (q2, s2) = O.quantize_mxfp4(w1e), O.quantize_mxfp4(w2e)
        np.testing.assert_array_equal(layer.w1_scale[e * twoI:(e + 1) * twoI].cpu().numpy(), s1)
        np.testing.assert_array_equal(layer.w2_scale[e * H:(e + 1) * H].cpu().numpy(), s2)
        d1, d2 = O.dequantize_mxfp4(q1, s1), O.dequantize_mxfp4(q2, s2)
    np.testing.assert_array_equal(layer.w1[e * twoI:(e + 1) * twoI].cpu().numpy(), q1)
    np.testing.assert_array_equal(layer.w2[e * H:(e + 1) * H].cpu().numpy(), q2)
    return d1, d2


def _oracle_tokens(cfg, x_rows):
    if cfg.dtype == O.DTYPE_BF16:
        return x_rows
    if cfg.dtype == O.DTYPE_FP8_BLOCK128:
        return O.dequantize_fp8_block(*O.quantize_fp8_block(x_rows, 1, 128), 1, 128)
    return O.dequantize_mxfp8(*O.quantize_mxfp8(x_rows))


_DEQ = {}          # dequantised experts of the current weight set: (weights key, e) -> (w1_hat, w2_hat)


def _experts_hat(cfg, layer, inp, experts, wkey):
    """The oracle's (dequantised) weights of each expert in `experts`, with the
    GPU's weight codes checked bit for bit against the oracle's quantisation
    (FP8 / MX). Experts are prepared in a thread pool (the float64 numpy
    quantisers release the GIL) and kept for later calls on the same weights."""
    from concurrent.futures import ThreadPoolExecutor
    if any(k[0] != wkey for k in _DEQ):
        _DEQ.clear()
    todo = [e for e in dict.fromkeys(experts) if (wkey, e) not in _DEQ]

    def one(e):
        return e, _oracle_expert(cfg, layer, e, to_f64(inp.w1[e]), to_f64(inp.w2[e]))

    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1, len(todo) or 1))) as ex:
        for e, wh in ex.map(one, todo):
            _DEQ[(wkey, e)] = wh
    return {e: _DEQ[(wkey, e)] for e in experts}


def _rows(t, idx):
    """Rows idx (numpy ints) of tensor t, on the host."""
    return t[torch.from_numpy(np.asarray(idx, np.int64)).to(t.device)].cpu()


def _sampled_compare(name, n_experts=4, rows_per_expert=3, n_tokens=0, inp=None, block_m=None, seed=0):
    """The forward of a full-size workload (name or Config) in the launch
    configuration the benchmark uses (or block_m): every routing and layout
    output in full; Y rows of n_experts experts (the most loaded one first),
    the first, last and rows_per_expert random rows of each, by the oracle one
    row at a time; the combine at full size as a property of the kernel's own
    Y and weights; n_tokens random tokens plus the first and last, whole,
    through the oracle. inp: inputs (host or device tensors); default the
    host-drawn ones of the workload."""
    cfg = get_config(name) if isinstance(name, str) else name
    if inp is None:
        inp = _inputs_cached(cfg)
    wkey = (cfg.cfg_id, cfg.E, cfg.H, cfg.I, cfg.w_std, inp.w1.device.type, seed)
    say("forward full-size sampled", cfg.name, cfg.T, block_m)
    layer, plan, out = _run(cfg, inp, block_m)
    logits = inp.logits.cpu().numpy()
    # every routing and layout output is compared in full
    rid, rw = O.route_with_shared(logits, cfg.k, cfg.score, cfg.n_shared)
    np.testing.assert_array_equal(plan.ids.cpu().numpy(), rid)
    assert_route_weights(plan.w.cpu().numpy(), rw)
    counts, offsets, sorted_ids, tile_expert, num_tiles = O.align_sort(rid, cfg.E_total, plan.block_m)
    np.testing.assert_array_equal(plan.sort.counts.cpu().numpy(), counts)
    np.testing.assert_array_equal(plan.sort.offsets.cpu().numpy(), offsets)
    assert int(plan.sort.num_tiles.item()) == num_tiles
    np.testing.assert_array_equal(plan.sort.sorted_ids.cpu().numpy()[:len(sorted_ids)], sorted_ids)
    np.testing.assert_array_equal(plan.sort.tile_expert.cpu().numpy()[:len(tile_expert)], tile_expert)
    rng = np.random.default_rng(seed)
    nonempty = np.flatnonzero(counts)
    experts = [int(np.argmax(counts))] + [int(e) for e in rng.choice(nonempty, min(n_experts, len(nonempty)),
                                                                     replace=False)]
    experts = list(dict.fromkeys(experts))[:n_experts]
    kk = cfg.k + cfg.n_shared
    toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, n_tokens, replace=False)])) \
        if n_tokens else np.zeros(0, np.int64)
    hat = _experts_hat(cfg, layer, inp, experts + sorted({int(e) for t in toks for e in rid[t]}), wkey)
    # sampled rows of Y, each evaluated by the oracle on its own
    assigned, refs = [], []
    for e in experts:
        seg = sorted_ids[offsets[e]:offsets[e] + counts[e]]
        pick = np.unique(np.concatenate([[seg[0], seg[-1]], rng.choice(seg, min(rows_per_expert, len(seg)),
                                                                       replace=False)]))
        w1h, w2h = hat[e]
        xr = _oracle_tokens(cfg, to_f64(_rows(inp.x, pick // kk)))
        refs += [O.assignment_forward(xr[i], w1h, w2h, cfg.dtype, cfg.act) for i in range(len(pick))]
        assigned += list(pick)
    got = f64(_rows(plan.y, assigned))
    ref = np.stack(refs)
    assert rel_fro(got, ref) <= TOL_FRO[cfg.dtype]
    assert min_row_cos(got, ref) >= TOL_COS
    # the combine at full size, as a property of the kernel's own Y and weights
    ctoks = rng.choice(cfg.T, min(cfg.T, 256), replace=False)
    yk = f64(plan.y.view(cfg.T, kk, cfg.H)[torch.from_numpy(ctoks).to(out.device)].reshape(-1, cfg.H))
    yk = yk.reshape(len(ctoks), kk, cfg.H)
    wk = plan.w.cpu().numpy()[ctoks].astype(np.float64)
    assert_within_rounding(f64(_rows(out, ctoks)), O.combine(yk.reshape(-1, cfg.H), wk),
                           kk * U32 * np.abs(wk[:, :, None] * yk).sum(1), min_exact=0.98)
    assert torch.isfinite(out.float()).all()
    # whole tokens through the oracle
    if n_tokens:
        w1 = {e: hat[e][0] for e in hat}
        w2 = {e: hat[e][1] for e in hat}
        x = _oracle_tokens(cfg, to_f64(_rows(inp.x, toks)))
        ref = np.stack([O.token_forward(x[i], w1, w2, rid[t], rw[t], cfg.dtype, cfg.act) for i, t in enumerate(toks)])
        got = f64(_rows(out, toks))
        assert rel_fro(got, ref) <= TOL_FRO[cfg.dtype]
        assert min_row_cos(got, ref) >= TOL_COS
    return layer, plan, out


@pytest.mark.parametrize("name", ["qwen3_30b_a3b_bf16", "qwen3_30b_a3b_bf16_zipf", "llama4_scout_bf16"])
def test_full_size_bf16_sampled(name):
    _sampled_compare(name, n_experts=4, n_tokens=6)


@pytest.mark.parametrize("T,E,k,S", [(64, 8, 2, 1), (129, 16, 4, 2), (1, 4, 2, 1), (300, 32, 8, 1)])
def test_shared_experts_forward_small(T, E, k, S):
    cfg = get_config("qwen3_30b_a3b_bf16_shared").with_(T=T, H=256, E=E, k=k, I=128, n_shared=S, w_std=0.05)
    _full_compare(cfg, make_inputs(cfg, seed=T + 11))


def test_shared_experts_full_size_sampled():
    # the most loaded expert is the shared one (every token): sampled first
    _sampled_compare("qwen3_30b_a3b_bf16_shared", n_experts=4, n_tokens=6)


@pytest.mark.parametrize("T,H,E,k,I", [(64, 256, 8, 2, 128), (129, 384, 16, 4, 200), (1, 256, 4, 2, 128),
                                       (300, 2688, 32, 6, 1856)])
def test_relu2_forward_small(T, H, E, k, I):
    cfg = get_config("nemotron_relu2_bf16").with_(T=T, H=H, E=E, k=k, I=I, w_std=0.05)
    _full_compare(cfg, make_inputs(cfg, seed=T + 7))


def test_relu2_full_size_sampled():
    _sampled_compare("nemotron_relu2_bf16", n_experts=4, n_tokens=6)


@pytest.mark.parametrize("name", P5_GRID)
def test_parameter_grid_sampled(name):
    """Every shape of the BF16 parameter grid (T = 8192, D = H = I in {2048,
    4096}, E in 8..128, top-K in 1..8), on the inputs the grid sweep of the
    benchmark times: drawn on the GPU with torch's seeded generator (drawing
    the 4096-wide shapes' weights on the host would take minutes each), then
    copied to the host for the oracle. Compared like the named workloads."""
    cfg = get_config(name)
    inp = make_inputs_device(cfg, "cuda:0")
    _sampled_compare(cfg, n_experts=3, n_tokens=2, inp=inp)
    del inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["qwen3_30b_a3b_bf16", "llama4_scout_bf16"])
@pytest.mark.parametrize("T", [1024, 2048, 4096, 16384])
def test_token_sweep_sampled(name, T):
    """The token-count sweep of the two named BF16 shapes (T = 8192 is the
    workload itself, above): each token count picks its own row tile."""
    _sampled_compare(get_config(name).with_(T=T), n_experts=4, n_tokens=4)


def test_qwen3_ragged_tokens_full_size():
    """T = 8191 on the full Qwen3-30B-A3B shape: a token count that is no
    multiple of anything, so the last tiles and the combine have ragged ends."""
    _sampled_compare(get_config("qwen3_30b_a3b_bf16").with_(T=8191), n_experts=4, n_tokens=6)


@pytest.mark.parametrize("T,block_m", [(256, None), (512, None), (1024, None), (4096, None), (1024, 32)])
def test_fp8_share_token_counts(T, block_m):
    """The FP8 64-expert H 7168 shape at the token counts where the row-tile
    rule picks 64-, 128- and 256-row tiles (the weight walk of each exceeds
    4 MB, so the grouped task order runs), and with 32-row tiles forced."""
    cfg = get_config("fp8_block128_share").with_(T=T)
    if block_m is None:
        assert M.moe_pick_block_m(cfg.dtype, T, cfg.k, cfg.E, cfg.H, cfg.I) == \
            {256: 64, 512: 128, 1024: 128, 4096: 256}[T]
    _sampled_compare(cfg, n_experts=4, n_tokens=2, block_m=block_m)


@pytest.mark.parametrize("name", ["fp8_block128_share", "mxfp4_moe_t128", "mxfp4_moe_t1024", "mxfp4_moe_t8192",
                                  "mxfp4_moe_t16384"])
def test_full_size_scaled_sampled(name):
    _sampled_compare(name, n_experts=4, n_tokens=6)


CANARY_CASES = [(O.DTYPE_BF16, 300, 16, 4, 256, 136, 32), (O.DTYPE_BF16, 700, 8, 2, 512, 256, 256),
                (O.DTYPE_FP8_BLOCK128, 257, 16, 4, 512, 256, 64), (O.DTYPE_MXFP4W_MXFP8A, 129, 64, 10, 512, 256, 32)]


@pytest.mark.parametrize("dtype,T,E,k,H,I,bm", CANARY_CASES)
def test_forward_leaves_slack_untouched(dtype, T, E, k, H, I, bm):
    """Every buffer of the forward is followed by a band of canary bytes, and
    the sorted-row buffers' rows past num_tiles * block_m hold canaries too:
    no kernel writes outside the rows the C ABI says it writes (GEMM1: rows
    < num_tiles * block_m of h and h_scale; GEMM2: rows < T * k of y; the
    combine: rows < T of out; align_sort: cap rows of sorted_ids, cap /
    block_m of tile_expert, E counts and E + 1 offsets)."""
    cfg = get_config("tiny_bf16").with_(T=T, H=H, E=E, k=k, I=I, dtype=dtype, w_std=0.05)
    inp = make_inputs(cfg, seed=T)
    say("forward canaries", dtype, T, E, k, H, I, bm)
    layer = M.MoeLayer(cfg.dtype, cuda(inp.w1), cuda(inp.w2), cfg.k, cfg.score)
    plan = layer.plan(T, block_m=bm)
    can = 0x6B

    def banded(t, extra_rows=16):
        big = torch.empty((t.shape[0] + extra_rows,) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)
        big.view(torch.uint8).fill_(can)
        return big

    bufs = {}
    for name in ("h", "h_scale", "y", "out"):
        t = getattr(plan, name)
        if t is not None:
            bufs[name] = banded(t)
            setattr(plan, name, bufs[name][:t.shape[0]])
    for name in ("sorted_ids", "tile_expert", "counts", "offsets"):
        t = getattr(plan.sort, name)
        bufs[name] = banded(t)
        setattr(plan.sort, name, bufs[name][:t.shape[0]])
    out = layer(cuda(inp.x), cuda(inp.logits), plan)
    torch.cuda.synchronize()
    rows = int(plan.sort.num_tiles.item()) * bm
    cap = plan.sort.cap
    lim = {"h": rows, "h_scale": rows, "y": T * k, "out": T, "sorted_ids": cap, "tile_expert": cap // bm,
           "counts": E, "offsets": E + 1}
    for name, big in bufs.items():
        tail = big[lim[name]:].contiguous().view(torch.uint8)
        assert bool((tail == can).all().item()), f"{name}: bytes written past row {lim[name]}"
    ref = O.moe_forward(inp.logits.numpy(), to_f64(inp.x), to_f64(inp.w1), to_f64(inp.w2), cfg.k, cfg.score,
                        cfg.dtype, block_m=bm)
    got = f64(out)
    assert rel_fro(got, ref["out"]) <= TOL_FRO[cfg.dtype]
    assert min_row_cos(got, ref["out"]) >= TOL_COS


@pytest.mark.parametrize("dtype", [O.DTYPE_FP8_BLOCK128, O.DTYPE_MXFP4W_MXFP8A])
@pytest.mark.parametrize("T,H,E,k,I", [(64, 256, 8, 2, 128), (129, 384, 16, 4, 256), (1, 256, 4, 2, 128),
                                       (300, 1024, 32, 8, 512), (257, 2560, 64, 10, 640)])
def test_scaled_forward_small(dtype, T, H, E, k, I):
    cfg = get_config("tiny_bf16").with_(T=T, H=H, E=E, k=k, I=I, dtype=dtype, w_std=0.05)
    _full_compare(cfg, make_inputs(cfg, seed=T + dtype))
