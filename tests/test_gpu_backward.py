"""GPU training step of the BF16 SwiGLU layer (forward with saved
pre-activations, then every backward call through the C ABI) against the
oracle's backward, on every element of every stored intermediate and
gradient.

Tolerances. Each bf16 intermediate (gu, dY, dGU, dx rows, dx) is the RN
rounding of a value the kernel accumulates in fp32 and the oracle in fp64, so
the two differ by at most one bf16 step wherever the fp32 error crosses a
rounding boundary, plus what earlier such flips carry downstream: relative
Frobenius error <= 5e-3 (one step is 2^-8 relative; only a small fraction of
elements flips). The fp32 outputs (dw, dW1, dW2) inherit the same flips in
their bf16 operands: relative Frobenius <= 5e-3. dlogits subtracts the
weighted mean of dw (softmax), which cancels: judged against its largest
element (atol 1e-2 of max) and by relative Frobenius <= 1e-2.

Beside those whole-tensor bounds, every stage is checked element by element
on the small shapes (_stagewise): the oracle stage is fed the GPU's own inputs
of that stage, so the only difference left is the kernel's fp32 arithmetic
(bounded by n 2^-24 times the sum of the magnitudes of the n terms) and one
storage rounding.
"""
import numpy as np
import pytest
import torch

import mixture_experts_routed_top_amd as M
from oracle import moe as O
from oracle import formats as F
from workloads import get_config, make_dout, make_inputs, to_f64
from tests.gpu_util import U32, assert_within_rounding, cuda, f64, rel_fro, say

pytestmark = pytest.mark.gpu

TOL = 5e-3
TOL_DLOGITS = 1e-2


def _train_step(cfg, inp, dout):
    layer = M.MoeLayer(M.DTYPE_BF16, cuda(inp.w1), cuda(inp.w2), cfg.k, cfg.score, n_shared=cfg.n_shared)
    plan = layer.plan(cfg.T, train=True)
    x = cuda(inp.x)
    out = layer.forward_train(x, cuda(inp.logits), plan)
    tb = layer.backward(x, cuda(dout), plan)
    torch.cuda.synchronize()
    return layer, plan, out, tb


def _per_expert_abs(a, w, tile_expert, nt, bm, transpose):
    """sum of |a[r]| |W[e]| per sorted row r of expert e (the magnitude that
    bounds an fp32 sum over the row's products): |a| @ |W[e]|.T or |a| @ |W[e]|."""
    out = np.zeros((nt * bm, w.shape[1] if transpose else w.shape[2]))
    for t in range(nt):
        e = tile_expert[t]
        blk = np.abs(a[t * bm:(t + 1) * bm])
        out[t * bm:(t + 1) * bm] = blk @ (np.abs(w[e]).T if transpose else np.abs(w[e]))
    return out


def _assert_fp32_close(got, ref, delta, what):
    """An fp32 result within delta (the bound of its fp32 arithmetic) plus
    its own final rounding of the exact value ref, element by element."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    lim = delta + U32 * np.abs(ref) + 1e-37
    bad = np.abs(got - ref) > lim
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} elements beyond the bound"


def _stagewise(cfg, inp, dout, plan, tb, ref):
    """Every stored intermediate and gradient against the oracle stage that
    produces it, fed the GPU's own inputs of that stage, element by element:
    within the fp32 arithmetic bound of the kernel's sums plus one storage
    rounding (bf16 values: assert_within_rounding; fp32 values: one fp32
    rounding). This pins single wrong elements that a Frobenius norm hides."""
    bm, kk = 256, cfg.k + cfg.n_shared
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E + cfg.n_shared
    A = T * kk
    nt = int(ref["num_tiles"])
    rows = nt * bm
    sid, te = ref["sorted_ids"], ref["tile_expert"]
    x, w1, w2, d = to_f64(inp.x), to_f64(inp.w1), to_f64(inp.w2), to_f64(dout)
    # forward: gu = bf16(g, u), h = bf16(silu(g) u), y = bf16(h W2^T)
    xs, g, u = O.gate_up_rows(x, w1, sid, te, nt, bm, kk)
    _, ga, ua = O.gate_up_rows(np.abs(x), np.abs(w1), sid, te, nt, bm, kk)
    gu = f64(tb.gu[:rows])
    assert_within_rounding(gu, F.round_bf16(np.concatenate([g, u], axis=1)),
                           np.concatenate([H * U32 * ga, H * U32 * ua], axis=1), min_exact=0.99)
    sig = 1.0 / (1.0 + np.exp(-np.clip(g, -700, 700)))
    dg, du = H * U32 * ga, H * U32 * ua
    delta_h = 1.1 * dg * (np.abs(u) + du) + np.abs(g * sig) * du + 8 * U32 * np.abs(g * sig * u)
    h = f64(plan.h[:rows])
    assert_within_rounding(h, F.round_bf16(O.silu(g) * u), delta_h, min_exact=0.99)
    y = f64(plan.y[:A])
    y_ref = O.grouped_gemm_down(h, w2, sid, te, nt, bm, A)
    y_abs = O.grouped_gemm_down(np.abs(h), np.abs(w2), sid, te, nt, bm, A)
    assert_within_rounding(y, y_ref, 1.01 * I * U32 * y_abs, min_exact=0.99)
    # combine backward: dy = bf16(w dout) (one fp32 product), dw = dout . y (H-term fp32 sum)
    w = plan.w.cpu().numpy().astype(np.float64)
    dy_ref, dw_ref = O.combine_backward(d, w, y, sid, nt, bm)
    dy_abs, dw_abs = O.combine_backward(np.abs(d), np.abs(w), np.abs(y), sid, nt, bm, exact=True)
    dy = f64(tb.dy[:rows])
    assert_within_rounding(dy, dy_ref, U32 * dy_abs, min_exact=0.99)
    dwg = tb.dw.cpu().numpy().astype(np.float64)
    _assert_fp32_close(dwg, dw_ref, H * U32 * dw_abs, "dw")
    # router backward from the GPU's w and dw
    ids = plan.ids.cpu().numpy()
    k = cfg.k
    dl_ref = O.route_backward(w[:, :k], ids[:, :k], dwg[:, :k], cfg.E, cfg.score).astype(np.float64)
    if cfg.score == O.SCORE_SOFTMAX:
        sabs = (np.abs(w[:, :k]) * np.abs(dwg[:, :k])).sum(1, keepdims=True)
        dl_d = 2 * np.abs(w[:, :k]) * ((k + 2) * U32 * (np.abs(dwg[:, :k]) + sabs))
    else:
        dl_d = 4 * U32 * np.abs(dwg[:, :k] * w[:, :k])
    delta_dl = np.zeros((T, cfg.E))
    np.put_along_axis(delta_dl, ids[:, :k].astype(np.int64), dl_d, axis=1)
    _assert_fp32_close(tb.dlogits.cpu().numpy(), dl_ref, delta_dl, "dlogits")
    # dGU from the GPU's dy and gu: dh = dy W2[e] (H-term fp32 sum), then the SwiGLU derivative
    dgu = f64(tb.dgu[:rows])
    dgu_ref = O.swiglu_backward(dy, w2, gu, te, nt, bm)
    dh_abs = H * U32 * _per_expert_abs(dy, w2, te, nt, bm, transpose=False)
    gs, us = gu[:, :I], gu[:, I:]
    s_ = 1.0 / (1.0 + np.exp(-gs))
    fac_g = np.abs(us * s_ * (1.0 + gs * (1.0 - s_)))
    fac_u = np.abs(gs * s_)
    dgu_exact = O.swiglu_backward(dy, w2, gu, te, nt, bm, exact=True)
    delta_dgu = np.concatenate([dh_abs * fac_g, dh_abs * fac_u], axis=1) + 16 * U32 * np.abs(dgu_exact)
    assert_within_rounding(dgu, dgu_ref, delta_dgu, min_exact=0.98)
    # dx rows from the GPU's dGU (2I-term fp32 sums), dx = bf16 of the fp32 slot sum
    dxr = f64(tb.dx_rows[:A])
    dxr_ref = O.dx_rows_backward(dgu, w1, sid, te, nt, bm, A)
    dxr_abs = O.dx_rows_backward(np.abs(dgu), np.abs(w1), sid, te, nt, bm, A, exact=True)
    assert_within_rounding(dxr, dxr_ref, 2 * I * U32 * dxr_abs, min_exact=0.99)
    ones = np.ones((T, kk))
    dx_ref = O.combine(dxr, ones)
    dx_abs = np.abs(dxr).reshape(T, kk, H).sum(1)
    assert_within_rounding(f64(tb.dx), dx_ref, kk * U32 * dx_abs, min_exact=0.99)
    # weight gradients from the GPU's h, dy, dgu and the gathered token rows (fp32 sums over each expert's rows)
    counts = np.bincount(ids.reshape(-1), minlength=E).astype(np.float64)
    for name, p_rows, q_rows in (("dw2", h, dy), ("dw1", xs, dgu)):
        wref = O.weight_grad(p_rows, q_rows, sid, te, nt, bm, A, E)
        wabs = O.weight_grad(np.abs(p_rows), np.abs(q_rows), sid, te, nt, bm, A, E)
        got = getattr(tb, name).cpu().numpy()
        _assert_fp32_close(got, wref, counts[:, None, None] * U32 * wabs, name)


def _check(cfg, seed=0, inp=None):
    inp = inp or make_inputs(cfg, seed=seed)
    dout = make_dout(cfg, seed)
    say("backward", cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.score, cfg.n_shared)
    layer, plan, out, tb = _train_step(cfg, inp, dout)
    ref = O.moe_backward(inp.logits.numpy(), to_f64(inp.x), to_f64(inp.w1), to_f64(inp.w2), to_f64(dout), cfg.k,
                         cfg.score, block_m=256, n_shared=cfg.n_shared)
    # routing and layout: exact
    np.testing.assert_array_equal(plan.ids.cpu().numpy(), ref["ids"])
    nt = int(plan.sort.num_tiles.item())
    assert nt == ref["num_tiles"]
    rows = nt * 256
    np.testing.assert_array_equal(plan.sort.sorted_ids.cpu().numpy()[:rows], ref["sorted_ids"][:rows])
    # forward intermediates
    assert rel_fro(f64(tb.gu[:rows]), ref["gu"]) <= TOL
    assert rel_fro(f64(plan.h[:rows]), ref["h"]) <= TOL
    assert rel_fro(f64(plan.y), ref["y"]) <= TOL
    # backward
    assert rel_fro(f64(tb.dy[:rows]), ref["dy"]) <= TOL
    assert rel_fro(tb.dw.cpu().numpy(), ref["dw"]) <= TOL
    dl, dl_ref = tb.dlogits.cpu().numpy().astype(np.float64), ref["dlogits"]
    assert rel_fro(dl, dl_ref) <= TOL_DLOGITS
    np.testing.assert_allclose(dl, dl_ref, rtol=0, atol=TOL_DLOGITS * max(np.abs(dl_ref).max(), 1e-30))
    # unselected experts carry exactly zero
    sel = np.zeros_like(dl_ref, dtype=bool)
    np.put_along_axis(sel, ref["ids"][:, :cfg.k].astype(np.int64), True, axis=1)
    assert np.all(dl[~sel] == 0)
    assert rel_fro(f64(tb.dgu[:rows]), ref["dgu"]) <= TOL
    assert rel_fro(f64(tb.dx_rows), ref["dx_rows"]) <= TOL
    assert rel_fro(f64(tb.dx), ref["dx"]) <= TOL
    dw1, dw2 = tb.dw1.cpu().numpy(), tb.dw2.cpu().numpy()
    assert rel_fro(dw1, ref["dw1"]) <= TOL
    assert rel_fro(dw2, ref["dw2"]) <= TOL
    # experts without rows have exactly zero weight gradients
    counts = np.bincount(ref["ids"].reshape(-1), minlength=layer.E)
    for e in np.nonzero(counts == 0)[0]:
        assert not dw1[e].any() and not dw2[e].any()
    _stagewise(cfg, inp, dout, plan, tb, ref)
    return ref


@pytest.mark.parametrize("T,H,E,k,I,score", [
    (200, 256, 6, 2, 192, O.SCORE_SOFTMAX),     # I below one 256-wide tile
    (333, 320, 8, 3, 200, O.SCORE_SIGMOID),     # ragged H and I tails, two m tiles of H
    (700, 256, 4, 2, 320, O.SCORE_SOFTMAX),     # several 256-row tiles per expert, two m tiles of I
    (100, 512, 4, 1, 256, O.SCORE_SOFTMAX),     # k = 1
    (1, 256, 8, 2, 128, O.SCORE_SOFTMAX),       # one token
])
def test_backward_small(T, H, E, k, I, score):
    cfg = get_config("tiny_bf16").with_(T=T, H=H, E=E, k=k, I=I, score=score, w_std=0.05)
    _check(cfg, seed=T)


def test_backward_shared_expert():
    cfg = get_config("tiny_bf16").with_(T=150, H=256, E=6, k=2, I=128, n_shared=1, w_std=0.05)
    ref = _check(cfg, seed=5)
    assert ref["ids"].shape[1] == 3


def test_backward_one_expert_takes_all():
    cfg = get_config("tiny_bf16").with_(T=300, H=256, E=8, k=1, I=128, w_std=0.05)
    inp = make_inputs(cfg, seed=3)
    inp.logits[:] = -1.0
    inp.logits[:, 5] = 2.0         # every token -> expert 5; the other experts stay empty
    _check(cfg, seed=3, inp=inp)


def test_backward_deterministic():
    cfg = get_config("tiny_bf16").with_(T=513, H=256, E=16, k=4, I=128, w_std=0.05)
    inp, dout = make_inputs(cfg, seed=9), make_dout(cfg, 9)
    say("backward determinism")
    a = _train_step(cfg, inp, dout)[3]
    b = _train_step(cfg, inp, dout)[3]
    for name in ("dx", "dlogits", "dw1", "dw2"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name


@pytest.mark.parametrize("name", ["qwen3_30b_a3b_bf16", "llama4_scout_bf16"])
def test_backward_full_size_sampled(name):
    """The Qwen3-30B-A3B- and Llama 4 Scout-shaped layers at T = 8192, in the
    launch configuration the backward benchmark times: routing and layout
    compared in full; dx, dw and dlogits on sampled tokens, and dW1 / dW2 of
    the most and the least loaded expert, each from the oracle run on just
    the tokens that determine them (a token's gradients depend on that token
    alone; an expert's weight gradients on the tokens routed to it)."""
    cfg = get_config(name)
    inp = make_inputs(cfg)
    dout = make_dout(cfg, 0)
    say("backward full-size sampled", cfg.name)
    layer, plan, out, tb = _train_step(cfg, inp, dout)
    logits = inp.logits.numpy()
    rid, _ = O.route(logits, cfg.k, cfg.score)
    np.testing.assert_array_equal(plan.ids.cpu().numpy(), rid)
    counts, offsets, sorted_ids, tile_expert, num_tiles = O.align_sort(rid, cfg.E, 256)
    np.testing.assert_array_equal(plan.sort.sorted_ids.cpu().numpy()[:len(sorted_ids)], sorted_ids)
    np.testing.assert_array_equal(plan.sort.offsets.cpu().numpy(), offsets)
    x64, w1, w2, d64 = to_f64(inp.x), to_f64(inp.w1), to_f64(inp.w2), to_f64(dout)

    def oracle_on(tokens):
        return O.moe_backward(logits[tokens], x64[tokens], w1, w2, d64[tokens], cfg.k, cfg.score)

    rng = np.random.default_rng(1)
    toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, 30, replace=False)]))
    ref = oracle_on(toks)
    assert rel_fro(f64(tb.dx[torch.from_numpy(toks).to(tb.dx.device)]), ref["dx"]) <= TOL
    assert rel_fro(tb.dw.cpu().numpy()[toks], ref["dw"]) <= TOL
    dl = tb.dlogits.cpu().numpy().astype(np.float64)[toks]
    assert rel_fro(dl, ref["dlogits"]) <= TOL_DLOGITS
    np.testing.assert_allclose(dl, ref["dlogits"], rtol=0, atol=TOL_DLOGITS * np.abs(ref["dlogits"]).max())
    del ref

    nonempty = np.flatnonzero(counts)
    for e in (int(nonempty[np.argmax(counts[nonempty])]), int(nonempty[np.argmin(counts[nonempty])])):
        sub = np.flatnonzero((rid == e).any(axis=1))
        say("backward full-size expert", e, len(sub))
        ref = oracle_on(sub)
        assert rel_fro(tb.dw1[e].cpu().numpy(), ref["dw1"][e]) <= TOL
        assert rel_fro(tb.dw2[e].cpu().numpy(), ref["dw2"][e]) <= TOL
        del ref
