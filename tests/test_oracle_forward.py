"""Pins for the oracle's GEMM1 + SwiGLU, GEMM2, combine and whole forward (CPU).

* a hand-worked one-token case (tests/golden/forward_tiny.txt);
* a pure-Python scalar brute force (explicit loops over tokens, slots,
  outputs and the reduction index) on tiny shapes, for all three dtypes;
* E = 1, k = 1 equals a dense SwiGLU MLP evaluated with torch in float64;
* equivariance under token permutation and expert relabelling;
* W2 * 2 doubles Y and out exactly; the padded layout (block_m) changes nothing.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import moe as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


def _case(T, H, E, k, I, seed, wstd=0.3):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.standard_normal((T, H)))
    w1 = _bf16(rng.standard_normal((E, 2 * I, H)) * wstd)
    w2 = _bf16(rng.standard_normal((E, H, I)) * wstd)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    return x, w1, w2, logits


def test_forward_golden():
    d = {}
    for line in open(os.path.join(GOLDEN, "forward_tiny.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            key, *vals = line.split()
            d[key] = [float(v) for v in vals]
    x = np.array(d["x"]).reshape(1, 2)
    w1 = np.array(d["w1"]).reshape(2, 2, 2)
    w2 = np.array(d["w2"]).reshape(2, 2, 1)
    r = O.moe_forward(np.array([d["logits"]], np.float32), x, w1, w2, int(d["k"][0]),
                      O.SCORE_SOFTMAX, O.DTYPE_BF16, block_m=16)
    assert r["ids"].tolist() == [[0]]
    assert r["h_val"][0, 0] == d["h"][0]
    assert r["y"][0].tolist() == d["y"]
    assert r["out"][0].tolist() == d["out"]


def _brute_forward(logits, x_hat, w1_hat, w2_hat, k, score, dtype):
    """Scalar loops; the storage roundings use the (separately pinned) codecs."""
    T, H = x_hat.shape
    E, twoI, _ = w1_hat.shape
    I = twoI // 2
    out = np.zeros((T, H))
    ys = np.zeros((T * k, H))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        sel = [float(logits[t, e]) for e in order]
        if score == O.SCORE_SOFTMAX:
            z = [math.exp(s - sel[0]) for s in sel]
            w = [float(np.float32(zi / sum(z))) for zi in z]
        else:
            w = [float(np.float32(1.0 / (1.0 + math.exp(-s)))) for s in sel]
        acc = [0.0] * H
        for j, e in enumerate(order):
            h = []
            for n in range(I):
                g = sum(x_hat[t, c] * w1_hat[e, n, c] for c in range(H))
                u = sum(x_hat[t, c] * w1_hat[e, I + n, c] for c in range(H))
                h.append(g / (1.0 + math.exp(-g)) * u)
            h = np.array([h])
            if dtype == O.DTYPE_BF16:
                hv = F.round_bf16(h)
            elif dtype == O.DTYPE_FP8_BLOCK128:
                hv = O.dequantize_fp8_block(*O.quantize_fp8_block(h, 1, 128), 1, 128)
            else:
                hv = O.dequantize_mxfp8(*O.quantize_mxfp8(h))
            for c in range(H):
                y = float(F.round_bf16(sum(hv[0, n] * w2_hat[e, c, n] for n in range(I))))
                ys[t * k + j, c] = y
                acc[c] += w[j] * y
        out[t] = F.round_bf16(np.array(acc))
    return ys, out


@pytest.mark.parametrize("dtype,H,I", [(O.DTYPE_BF16, 8, 4), (O.DTYPE_FP8_BLOCK128, 128, 128),
                                       (O.DTYPE_MXFP4W_MXFP8A, 64, 32)])
def test_forward_scalar_brute_force(dtype, H, I):
    T, E, k = (5, 4, 2) if dtype == O.DTYPE_BF16 else (3, 3, 2)
    x, w1, w2, logits = _case(T, H, E, k, I, seed=dtype + 1)
    r = O.moe_forward(logits, x, w1, w2, k, O.SCORE_SOFTMAX, dtype, block_m=16)
    if dtype == O.DTYPE_BF16:
        xh, w1h, w2h = x, w1, w2
    elif dtype == O.DTYPE_FP8_BLOCK128:
        xh = O.dequantize_fp8_block(*O.quantize_fp8_block(x, 1, 128), 1, 128)
        w1h = O.dequantize_fp8_block(*O.quantize_fp8_block(w1.reshape(-1, H), 128, 128), 128, 128).reshape(w1.shape)
        w2h = O.dequantize_fp8_block(*O.quantize_fp8_block(w2.reshape(-1, I), 128, 128), 128, 128).reshape(w2.shape)
    else:
        xh = O.dequantize_mxfp8(*O.quantize_mxfp8(x))
        w1h = O.dequantize_mxfp4(*O.quantize_mxfp4(w1.reshape(-1, H))).reshape(w1.shape)
        w2h = O.dequantize_mxfp4(*O.quantize_mxfp4(w2.reshape(-1, I))).reshape(w2.shape)
    ys, out = _brute_forward(logits, xh, w1h, w2h, k, O.SCORE_SOFTMAX, dtype)
    # identical roundings; only the float64 summation order differs
    np.testing.assert_allclose(r["y"], ys, rtol=2 ** -7, atol=1e-12)
    assert np.mean(r["y"] == ys) > 0.99
    np.testing.assert_allclose(r["out"], out, rtol=2 ** -7, atol=1e-12)


def test_forward_sigmoid_brute_force():
    x, w1, w2, logits = _case(6, 8, 4, 1, 4, seed=42)
    r = O.moe_forward(logits, x, w1, w2, 1, O.SCORE_SIGMOID, O.DTYPE_BF16, block_m=16)
    ys, out = _brute_forward(logits, x, w1, w2, 1, O.SCORE_SIGMOID, O.DTYPE_BF16)
    np.testing.assert_allclose(r["out"], out, rtol=2 ** -7, atol=1e-12)


def test_e1_k1_equals_dense_swiglu_mlp():
    T, H, I = 16, 64, 32
    x, w1, w2, logits = _case(T, H, 1, 1, I, seed=5)
    r = O.moe_forward(logits, x, w1, w2, 1, O.SCORE_SOFTMAX, O.DTYPE_BF16, block_m=16)
    assert np.all(r["w"] == 1.0)
    xt = torch.from_numpy(x)
    gate = xt @ torch.from_numpy(w1[0, :I]).T
    up = xt @ torch.from_numpy(w1[0, I:]).T
    h = torch.nn.functional.silu(gate) * up
    np.testing.assert_allclose(_unsort(r, r["h_val"], T), F.round_bf16(h.numpy()),
                               rtol=2 ** -8, atol=0)
    y = torch.from_numpy(F.round_bf16(h.numpy())) @ torch.from_numpy(w2[0]).T
    np.testing.assert_array_equal(r["out"], F.round_bf16(y.numpy()))


def _unsort(r, rows, T):
    """h rows in token order for k = 1."""
    out = np.zeros((T, rows.shape[1]))
    for pos, a in enumerate(r["sorted_ids"][:rows.shape[0]]):
        if a < T:
            out[a] = rows[pos]
    return out


def test_token_permutation_and_expert_relabelling_equivariance():
    T, H, E, k, I = 24, 32, 6, 2, 16
    x, w1, w2, logits = _case(T, H, E, k, I, seed=8)
    base = O.moe_forward(logits, x, w1, w2, k, O.SCORE_SOFTMAX, O.DTYPE_BF16)
    p = np.random.default_rng(1).permutation(T)
    r = O.moe_forward(logits[p], x[p], w1, w2, k, O.SCORE_SOFTMAX, O.DTYPE_BF16)
    np.testing.assert_array_equal(r["out"], base["out"][p])
    q = np.random.default_rng(2).permutation(E)            # new expert i is old expert q[i]
    r = O.moe_forward(logits[:, q], x, w1[q], w2[q], k, O.SCORE_SOFTMAX, O.DTYPE_BF16)
    np.testing.assert_array_equal(r["out"], base["out"])


def test_w2_scaling_and_block_m_invariance():
    T, H, E, k, I = 20, 32, 5, 2, 16
    x, w1, w2, logits = _case(T, H, E, k, I, seed=9)
    a = O.moe_forward(logits, x, w1, w2, k, O.SCORE_SOFTMAX, O.DTYPE_BF16, block_m=16)
    b = O.moe_forward(logits, x, w1, 2 * w2, k, O.SCORE_SOFTMAX, O.DTYPE_BF16, block_m=64)
    np.testing.assert_array_equal(b["y"], 2 * a["y"])
    np.testing.assert_array_equal(b["out"], 2 * a["out"])
    c = O.moe_forward(logits, x, w1, w2, k, O.SCORE_SOFTMAX, O.DTYPE_BF16, block_m=128)
    np.testing.assert_array_equal(c["y"], a["y"])


def test_gate_and_up_halves_are_not_interchangeable():
    # swapping the gate and up halves of W1 must change the result (silu is not symmetric)
    T, H, E, k, I = 8, 16, 2, 1, 8
    x, w1, w2, logits = _case(T, H, E, k, I, seed=10)
    a = O.moe_forward(logits, x, w1, w2, k, O.SCORE_SOFTMAX, O.DTYPE_BF16)
    sw = np.concatenate([w1[:, I:], w1[:, :I]], axis=1)
    b = O.moe_forward(logits, x, sw, w2, k, O.SCORE_SOFTMAX, O.DTYPE_BF16)
    assert not np.array_equal(a["out"], b["out"])


@pytest.mark.parametrize("dtype", [O.DTYPE_BF16, O.DTYPE_FP8_BLOCK128, O.DTYPE_MXFP4W_MXFP8A])
def test_token_forward_matches_moe_forward(dtype):
    T, H, E, k, I = 6, 128, 4, 2, 128
    x, w1, w2, logits = _case(T, H, E, k, I, seed=11 + dtype)
    r = O.moe_forward(logits, x, w1, w2, k, O.SCORE_SOFTMAX, dtype)
    if dtype == O.DTYPE_BF16:
        xh, w1h, w2h = x, w1, w2
    elif dtype == O.DTYPE_FP8_BLOCK128:
        xh = O.dequantize_fp8_block(r["xq"], r["xs"], 1, 128)
        w1h = O.dequantize_fp8_block(*O.quantize_fp8_block(w1.reshape(-1, H), 128, 128), 128, 128).reshape(w1.shape)
        w2h = O.dequantize_fp8_block(*O.quantize_fp8_block(w2.reshape(-1, I), 128, 128), 128, 128).reshape(w2.shape)
    else:
        xh = O.dequantize_mxfp8(r["xq"], r["xs"])
        w1h = O.dequantize_mxfp4(*O.quantize_mxfp4(w1.reshape(-1, H))).reshape(w1.shape)
        w2h = O.dequantize_mxfp4(*O.quantize_mxfp4(w2.reshape(-1, I))).reshape(w2.shape)
    for t in range(T):
        o = O.token_forward(xh[t], w1h, w2h, r["ids"][t], r["w"][t], dtype)
        np.testing.assert_allclose(o, r["out"][t], rtol=2 ** -7, atol=1e-12)


# ------------------------------------------------------------------ squared-ReLU (ungated) experts
def _relu2_case(T, H, E, k, I, seed, wstd=0.3):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.standard_normal((T, H)))
    w1 = _bf16(rng.standard_normal((E, I, H)) * wstd)
    w2 = _bf16(rng.standard_normal((E, H, I)) * wstd)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    return x, w1, w2, logits


def test_relu2_scalar_brute_force():
    """Explicit loops: h_n = max(sum_c x_c W1[e, n, c], 0)^2 stored bf16, then
    y = bf16(sum_n h_n W2[e, :, n]) and the weighted combine."""
    T, H, E, k, I = 5, 8, 4, 2, 6
    x, w1, w2, logits = _relu2_case(T, H, E, k, I, seed=21)
    r = O.moe_forward(logits, x, w1, w2, k, O.SCORE_SOFTMAX, O.DTYPE_BF16, act=O.ACT_RELU2)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        z = [math.exp(float(logits[t, e]) - float(logits[t, order[0]])) for e in order]
        w = [float(np.float32(zi / sum(z))) for zi in z]
        acc = [0.0] * H
        for j, e in enumerate(order):
            h = []
            for n in range(I):
                g = sum(x[t, c] * w1[e, n, c] for c in range(H))
                h.append(float(F.round_bf16(np.array([g * g if g > 0 else 0.0]))[0]))
            for c in range(H):
                y = float(F.round_bf16(np.array([sum(h[n] * w2[e, c, n] for n in range(I))]))[0])
                assert abs(r["y"][t * k + j, c] - y) <= 2 ** -7 * abs(y) + 1e-12
                acc[c] += w[j] * y
        np.testing.assert_allclose(r["out"][t], F.round_bf16(np.array(acc)), rtol=2 ** -7, atol=1e-12)


def test_relu2_e1_k1_equals_dense_relu2_mlp():
    T, H, I = 16, 64, 32
    x, w1, w2, logits = _relu2_case(T, H, 1, 1, I, seed=22)
    r = O.moe_forward(logits, x, w1, w2, 1, O.SCORE_SOFTMAX, O.DTYPE_BF16, act=O.ACT_RELU2)
    h = torch.relu(torch.from_numpy(x) @ torch.from_numpy(w1[0]).T) ** 2
    np.testing.assert_allclose(_unsort(r, r["h_val"], T), F.round_bf16(h.numpy()), rtol=2 ** -8, atol=0)
    y = torch.from_numpy(F.round_bf16(h.numpy())) @ torch.from_numpy(w2[0]).T
    np.testing.assert_array_equal(r["out"], F.round_bf16(y.numpy()))


def test_relu2_negative_preactivations_give_zero_h():
    # every pre-activation negative: h must be exactly 0 (no leak, no square of a negative)
    T, H, I = 8, 16, 8
    x = np.abs(_bf16(np.random.default_rng(3).standard_normal((T, H)))) + 0.5
    w1 = -np.abs(_bf16(np.random.default_rng(4).standard_normal((1, I, H)))) - 0.25
    w2 = _bf16(np.random.default_rng(5).standard_normal((1, H, I)))
    logits = np.zeros((T, 1), np.float32)
    r = O.moe_forward(logits, x, w1, w2, 1, O.SCORE_SOFTMAX, O.DTYPE_BF16, act=O.ACT_RELU2)
    assert np.all(r["h_val"] == 0.0) and np.all(r["out"] == 0.0)
    # and the squared branch: W1 -> -W1 makes every pre-activation positive
    r2 = O.moe_forward(logits, x, -w1, w2, 1, O.SCORE_SOFTMAX, O.DTYPE_BF16, act=O.ACT_RELU2)
    g = x @ (-w1[0]).T
    np.testing.assert_array_equal(_unsort(r2, r2["h_val"], T), F.round_bf16(g * g))


def test_relu2_flops():
    assert O.routed_flops(8192, 6, 2688, 1856, O.ACT_RELU2) == 4 * 8192 * 6 * 2688 * 1856
    assert O.routed_flops(8192, 6, 2688, 1856) == 6 * 8192 * 6 * 2688 * 1856


# ------------------------------------------------------------------ shared experts
def test_route_with_shared_appends_fixed_slots():
    logits = np.random.default_rng(0).standard_normal((7, 6)).astype(np.float32)
    ids, w = O.route_with_shared(logits, 2, O.SCORE_SOFTMAX, 3)
    rid, rw = O.route(logits, 2, O.SCORE_SOFTMAX)
    assert ids.shape == (7, 5) and w.shape == (7, 5)
    np.testing.assert_array_equal(ids[:, :2], rid)
    np.testing.assert_array_equal(w[:, :2], rw)
    np.testing.assert_array_equal(ids[:, 2:], np.tile([6, 7, 8], (7, 1)))
    assert np.all(w[:, 2:] == 1.0)


def test_shared_expert_adds_a_dense_mlp():
    """out = bf16( sum_j w_j y_j + y_shared ), y_shared = bf16 of the dense
    SwiGLU MLP of the shared weights (torch float64), y_j the routed rows."""
    T, H, E, k, I = 12, 32, 5, 2, 16
    x, w1, w2, logits = _case(T, H, E + 1, k, I, seed=31)
    logits = np.ascontiguousarray(logits[:, :E])     # the router scores the E routed experts only
    routed = O.moe_forward(logits, x, w1[:E], w2[:E], k, O.SCORE_SOFTMAX, O.DTYPE_BF16)
    shared = O.moe_forward(logits, x, w1, w2, k, O.SCORE_SOFTMAX, O.DTYPE_BF16, n_shared=1)
    xt = torch.from_numpy(x)
    hs = torch.nn.functional.silu(xt @ torch.from_numpy(w1[E, :I]).T) * (xt @ torch.from_numpy(w1[E, I:]).T)
    ys = F.round_bf16((torch.from_numpy(F.round_bf16(hs.numpy())) @ torch.from_numpy(w2[E]).T).numpy())
    yr = routed["y"].reshape(T, k, H)
    w = routed["w"].astype(np.float64)
    expect = F.round_bf16((w[:, :, None] * yr).sum(1) + ys)
    np.testing.assert_array_equal(shared["y"].reshape(T, k + 1, H)[:, :k], yr)
    np.testing.assert_array_equal(shared["y"].reshape(T, k + 1, H)[:, k], ys)
    np.testing.assert_array_equal(shared["out"], expect)


def test_wide_shared_expert_equals_two_narrow_ones():
    # a shared expert of width 2I is two of width I (its intermediate columns
    # split in two) up to the bf16 rounding of each half's Y row
    T, H, E, k, I = 10, 32, 4, 2, 8
    x, w1, w2, logits = _case(T, H, E, k, I, seed=32)
    rng = np.random.default_rng(33)
    g = _bf16(rng.standard_normal((2 * I, H)) * 0.3)
    u = _bf16(rng.standard_normal((2 * I, H)) * 0.3)
    d = _bf16(rng.standard_normal((H, 2 * I)) * 0.3)
    # one layer holds one I: the routed experts are zero-padded to width 2I there
    pad = lambda a, axis: np.concatenate([a, np.zeros_like(a)], axis=axis)
    w1r = np.concatenate([pad(w1[:, :I], 1), pad(w1[:, I:], 1)], axis=1)    # routed, zero-padded to 2I
    w2r = pad(w2, 2)
    wide_w1 = np.concatenate([w1r, np.concatenate([g, u])[None]], axis=0)
    wide_w2 = np.concatenate([w2r, d[None]], axis=0)
    a = O.moe_forward(logits, x, wide_w1, wide_w2, k, O.SCORE_SOFTMAX, O.DTYPE_BF16, n_shared=1)
    halves_w1 = np.stack([np.concatenate([g[:I], u[:I]]), np.concatenate([g[I:], u[I:]])])
    halves_w2 = np.stack([d[:, :I], d[:, I:]])
    narrow_w1 = np.concatenate([w1, halves_w1], axis=0)
    narrow_w2 = np.concatenate([w2, halves_w2], axis=0)
    b = O.moe_forward(logits, x, narrow_w1, narrow_w2, k, O.SCORE_SOFTMAX, O.DTYPE_BF16, n_shared=2)
    np.testing.assert_allclose(b["out"], a["out"], rtol=2 ** -6, atol=2 ** -6)   # one bf16 step of O(1) values
