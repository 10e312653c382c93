"""Pins for the oracle's backward of the BF16 SwiGLU routed forward (CPU).

* with the storage roundings dropped (exact=True) the oracle's gradients are
  the mathematical ones: compared with torch autograd in float64 on the plain
  forward, and with central finite differences of a scalar loss written out
  with loops;
* the routing-weight backward against torch autograd of the softmax over the
  selected logits and of the sigmoid;
* the rounded gradients stay within bf16-level error of the exact ones;
* shared experts: the shared slots carry no routing gradient.
"""
import numpy as np
import pytest
import torch

from oracle import moe as O


def _case(T, H, E, k, I, seed, wstd=0.3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    w1 = rng.standard_normal((E, 2 * I, H)) * wstd
    w2 = rng.standard_normal((E, H, I)) * wstd
    logits = rng.standard_normal((T, E)).astype(np.float32)
    dout = rng.standard_normal((T, H))
    return x, w1, w2, logits, dout


def _torch_grads(x, w1, w2, logits, dout, k, score):
    """Autograd of sum(out * dout) for the plain float64 forward with the
    oracle's top-k choice held fixed."""
    ids, _ = O.route(logits, k, score)
    xt = torch.tensor(x, requires_grad=True)
    w1t = torch.tensor(w1, requires_grad=True)
    w2t = torch.tensor(w2, requires_grad=True)
    lt = torch.tensor(logits.astype(np.float64), requires_grad=True)
    I = w1.shape[1] // 2
    out = []
    for t in range(x.shape[0]):
        sel = lt[t, torch.tensor(ids[t], dtype=torch.long)]
        wt = torch.softmax(sel, 0) if score == O.SCORE_SOFTMAX else torch.sigmoid(sel)
        acc = 0.0
        for j, e in enumerate(ids[t]):
            g = w1t[e, :I] @ xt[t]
            u = w1t[e, I:] @ xt[t]
            acc = acc + wt[j] * (w2t[e] @ (torch.nn.functional.silu(g) * u))
        out.append(acc)
    loss = (torch.stack(out) * torch.tensor(dout)).sum()
    loss.backward()
    return xt.grad.numpy(), w1t.grad.numpy(), w2t.grad.numpy(), lt.grad.numpy()


@pytest.mark.parametrize("score,k", [(O.SCORE_SOFTMAX, 2), (O.SCORE_SOFTMAX, 3), (O.SCORE_SIGMOID, 1)])
def test_exact_backward_equals_autograd(score, k):
    T, H, E, I = 7, 12, 5, 6
    x, w1, w2, logits, dout = _case(T, H, E, k, I, seed=k + 10 * score)
    r = O.moe_backward(logits, x, w1, w2, dout, k, score, exact=True)
    dx, dw1, dw2, dl = _torch_grads(x, w1, w2, logits, dout, k, score)
    # the routed weights are fp32 (route's storage point): relative 2^-24 each
    close = lambda a, b: np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-6 * np.abs(b).max())
    close(r["dx"], dx)
    close(r["dw1"], dw1)
    close(r["dw2"], dw2)
    # the routed weights are stored in fp32 and dlogits is fp32
    np.testing.assert_allclose(r["dlogits"], dl, rtol=1e-5, atol=1e-6)


def _loss(x, w1, w2, logits, dout, ids, score):
    """sum(out * dout) with explicit loops, the top-k choice given."""
    T, H = x.shape
    I = w1.shape[1] // 2
    total = 0.0
    for t in range(T):
        sel = [float(logits[t, e]) for e in ids[t]]
        if score == O.SCORE_SOFTMAX:
            z = [np.exp(s - max(sel)) for s in sel]
            wt = [zi / sum(z) for zi in z]
        else:
            wt = [1.0 / (1.0 + np.exp(-s)) for s in sel]
        for j, e in enumerate(ids[t]):
            for c in range(H):
                yc = 0.0
                for n in range(I):
                    g = sum(w1[e, n, q] * x[t, q] for q in range(H))
                    u = sum(w1[e, I + n, q] * x[t, q] for q in range(H))
                    yc += w2[e, c, n] * g / (1.0 + np.exp(-g)) * u
                total += dout[t, c] * wt[j] * yc
    return total


def test_exact_backward_finite_differences():
    T, H, E, k, I = 3, 4, 3, 2, 3
    x, w1, w2, logits, dout = _case(T, H, E, k, I, seed=5)
    logits = logits.astype(np.float64)
    r = O.moe_backward(logits, x, w1, w2, dout, k, O.SCORE_SOFTMAX, exact=True)
    ids = r["ids"]
    eps = 1e-6
    rng = np.random.default_rng(6)
    for name, arr, grad in (("x", x, r["dx"]), ("w1", w1, r["dw1"]), ("w2", w2, r["dw2"])):
        for _ in range(4):
            idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
            p, m = arr.copy(), arr.copy()
            p[idx] += eps
            m[idx] -= eps
            args = {"x": x, "w1": w1, "w2": w2}
            lp = _loss(**{**args, name: p}, logits=logits, dout=dout, ids=ids, score=O.SCORE_SOFTMAX)
            lm = _loss(**{**args, name: m}, logits=logits, dout=dout, ids=ids, score=O.SCORE_SOFTMAX)
            assert abs((lp - lm) / (2 * eps) - grad[idx]) <= 1e-6 * max(1.0, abs(grad[idx])), (name, idx)
    # a routed logit (selection unchanged by the small step)
    t, j = 1, 0
    e = int(ids[t, j])
    p, m = logits.copy(), logits.copy()
    p[t, e] += eps
    m[t, e] -= eps
    fd = (_loss(x, w1, w2, p, dout, ids, O.SCORE_SOFTMAX) - _loss(x, w1, w2, m, dout, ids, O.SCORE_SOFTMAX)) / (2 * eps)
    assert abs(fd - r["dlogits"][t, e]) <= 1e-5 * max(1.0, abs(fd))


@pytest.mark.parametrize("score", [O.SCORE_SOFTMAX, O.SCORE_SIGMOID])
def test_route_backward_against_autograd(score):
    rng = np.random.default_rng(7)
    T, E, k = 9, 6, 3 if score == O.SCORE_SOFTMAX else 1
    logits = rng.standard_normal((T, E))
    dw = rng.standard_normal((T, k))
    ids, w = O.route(logits.astype(np.float32), k, score)
    lt = torch.tensor(logits, requires_grad=True)
    sel = torch.gather(lt, 1, torch.tensor(ids, dtype=torch.long))
    wt = torch.softmax(sel, 1) if score == O.SCORE_SOFTMAX else torch.sigmoid(sel)
    (wt * torch.tensor(dw)).sum().backward()
    got = O.route_backward(w, ids, dw, E, score)
    np.testing.assert_allclose(got, lt.grad.numpy(), rtol=1e-5, atol=1e-6)
    unselected = np.ones((T, E), bool)
    np.put_along_axis(unselected, ids.astype(np.int64), False, axis=1)
    assert np.all(got[unselected] == 0)


def test_rounded_backward_close_to_exact():
    T, H, E, k, I = 16, 32, 4, 2, 16
    x, w1, w2, logits, dout = _case(T, H, E, k, I, seed=8)
    rb = lambda a: torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).double().numpy()
    x, w1, w2, dout = rb(x), rb(w1), rb(w2), rb(dout)
    a = O.moe_backward(logits, x, w1, w2, dout, k, O.SCORE_SOFTMAX, exact=True)
    b = O.moe_backward(logits, x, w1, w2, dout, k, O.SCORE_SOFTMAX)
    for key in ("dx", "dw1", "dw2"):
        rel = np.linalg.norm(b[key] - a[key]) / np.linalg.norm(a[key])
        assert rel < 2e-2, (key, rel)
    # block_m does not change a single bit of the rounded gradients
    c = O.moe_backward(logits, x, w1, w2, dout, k, O.SCORE_SOFTMAX, block_m=64)
    for key in ("dx", "dw1", "dw2", "dw", "dlogits"):
        np.testing.assert_array_equal(c[key], b[key])


def test_shared_slots_have_no_routing_gradient():
    T, H, E, k, I = 6, 8, 4, 2, 4
    x, w1, w2, logits, dout = _case(T, H, E + 1, k, I, seed=9)
    logits = np.ascontiguousarray(logits[:, :E])
    r = O.moe_backward(logits, x, w1, w2, dout, k, O.SCORE_SOFTMAX, n_shared=1, exact=True)
    assert r["dlogits"].shape == (T, E)
    # the shared expert's weight gradient is the dense MLP's: sum over every token
    xt = torch.tensor(x)
    w1s = torch.tensor(w1[E], requires_grad=True)
    w2s = torch.tensor(w2[E], requires_grad=True)
    hs = torch.nn.functional.silu(xt @ w1s[:I].T) * (xt @ w1s[I:].T)
    ((hs @ w2s.T) * torch.tensor(dout)).sum().backward()
    np.testing.assert_allclose(r["dw1"][E], w1s.grad.numpy(), rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(r["dw2"][E], w2s.grad.numpy(), rtol=1e-6, atol=1e-9)
