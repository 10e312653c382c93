"""Pins for the oracle's route and align_sort (CPU only).

route is checked against a brute-force Python sort, hand-worked cases in
tests/golden/route_tiny.txt, the closed forms of softmax / sigmoid, and the
equality "softmax over the k selected logits == softmax over all E
renormalised over the top k" evaluated with torch in float64.
align_sort is checked against brute force sorted(range(A), key=(expert, a)),
the hand-worked case in tests/golden/align_tiny.txt and its invariants.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import moe as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- route
def _golden_route_cases():
    cases = []
    for line in open(os.path.join(GOLDEN, "route_tiny.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        score, k, logits, ids, w = [p.strip() for p in line.split("|")]
        cases.append((O.SCORE_SOFTMAX if score == "softmax" else O.SCORE_SIGMOID, int(k),
                      [float(v) for v in logits.split()], [int(v) for v in ids.split()],
                      [eval(expr, {"exp": math.exp}) for expr in w.split(";")]))
    return cases


@pytest.mark.parametrize("case", _golden_route_cases())
def test_route_golden(case):
    score, k, logits, ids, w = case
    got_ids, got_w = O.route(np.array([logits], np.float32), k, score)
    assert got_ids[0].tolist() == ids
    np.testing.assert_array_equal(got_w[0], np.array(w, np.float64).astype(np.float32))


def _brute_route(row, k):
    return [e for e, _ in sorted(enumerate(row), key=lambda p: (-p[1], p[0]))][:k]


@pytest.mark.parametrize("E,k", [(4, 1), (8, 2), (16, 5), (33, 8), (64, 10)])
def test_route_brute_force_with_ties(E, k):
    rng = np.random.default_rng(E * 100 + k)
    # small integer logits force many exact ties
    logits = rng.integers(-3, 4, size=(50, E)).astype(np.float32)
    ids, w = O.route(logits, k, O.SCORE_SOFTMAX)
    for t in range(50):
        assert ids[t].tolist() == _brute_route(logits[t].tolist(), k)
        sel = [float(logits[t, e]) for e in ids[t]]
        z = [math.exp(v - sel[0]) for v in sel]
        ref = [zi / sum(z) for zi in z]
        np.testing.assert_array_equal(w[t], np.array(ref).astype(np.float32))


def test_route_softmax_equals_full_softmax_renormalised():
    rng = np.random.default_rng(7)
    logits = (rng.standard_normal((200, 128)) * 3).astype(np.float32)
    ids, w = O.route(logits, 8, O.SCORE_SOFTMAX)
    p = torch.softmax(torch.from_numpy(logits).double(), dim=1)
    topv, topi = torch.topk(p, 8, dim=1)
    assert np.array_equal(topi.numpy(), ids)          # no ties in continuous draws
    ref = (topv / topv.sum(dim=1, keepdim=True)).numpy()
    np.testing.assert_allclose(w, ref, rtol=2 ** -23, atol=0)
    # invariants: weights sum to one, are non-increasing
    np.testing.assert_allclose(w.astype(np.float64).sum(1), 1.0, atol=8 * 2 ** -24)
    assert np.all(np.diff(w.astype(np.float64), axis=1) <= 0)


def test_route_sigmoid_top1_closed_form():
    rng = np.random.default_rng(3)
    logits = (rng.standard_normal((100, 16)) * 4).astype(np.float32)
    ids, w = O.route(logits, 1, O.SCORE_SIGMOID)
    assert np.array_equal(ids[:, 0], logits.argmax(1))
    ref = torch.sigmoid(torch.from_numpy(logits.max(1)).double()).numpy().astype(np.float32)
    np.testing.assert_array_equal(w[:, 0], ref)


def test_route_rejects_bad_k():
    with pytest.raises(ValueError):
        O.route(np.zeros((2, 4), np.float32), 5)
    with pytest.raises(ValueError):
        O.route(np.zeros((2, 4), np.float32), 0)


# ----------------------------------------------------------------- align_sort
def _golden_align():
    d = {}
    for line in open(os.path.join(GOLDEN, "align_tiny.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        d[key] = [int(v) for v in vals]
    return d


def test_align_sort_golden():
    g = _golden_align()
    E, bm = g["E"][0], g["block_m"][0]
    ids = np.array(g["ids"], np.int32).reshape(-1, 2)
    counts, offsets, sorted_ids, tile_expert, num_tiles = O.align_sort(ids, E, bm)
    assert counts.tolist() == g["counts"]
    assert offsets.tolist() == g["offsets"]
    assert sorted_ids.tolist() == g["sorted_ids"]
    assert tile_expert.tolist() == g["tile_expert"]
    assert num_tiles == g["num_tiles"][0]


def _check_align(ids, E, bm):
    T, k = ids.shape
    A = T * k
    counts, offsets, sorted_ids, tile_expert, num_tiles = O.align_sort(ids, E, bm)
    flat = ids.reshape(-1).tolist()
    brute = sorted(range(A), key=lambda a: (flat[a], a))
    cap = O.sorted_capacity(T, k, E, bm)
    assert len(sorted_ids) == cap and cap % bm == 0
    assert counts.sum() == A                                  # sum of counts = T*k
    assert [a for a in sorted_ids.tolist() if a != A] == brute  # stable, a permutation
    assert offsets[0] == 0 and offsets[-1] <= cap
    assert num_tiles * bm == offsets[-1]
    for e in range(E):
        seg = sorted_ids[offsets[e]:offsets[e + 1]]
        pad = offsets[e + 1] - offsets[e] - counts[e]
        assert 0 <= pad < bm and (offsets[e + 1] - offsets[e]) % bm == 0
        assert all(flat[a] == e for a in seg[:counts[e]])
        assert np.all(seg[counts[e]:] == A)
        tiles = tile_expert[offsets[e] // bm:offsets[e + 1] // bm]
        assert np.all(tiles == e) and len(tiles) == -(-counts[e] // bm)
    assert np.all(sorted_ids[offsets[-1]:] == A)
    assert np.all(tile_expert[num_tiles:] == -1)


@pytest.mark.parametrize("T,E,k,bm", [(1, 4, 1, 16), (7, 8, 2, 16), (64, 8, 2, 16),
                                      (129, 16, 4, 32), (300, 128, 8, 64), (50, 512, 10, 16),
                                      (33, 3, 3, 256)])
def test_align_sort_brute_force_and_invariants(T, E, k, bm):
    rng = np.random.default_rng(T + E + k + bm)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _check_align(ids, E, bm)


def test_align_sort_all_to_one_expert_and_empty():
    ids = np.zeros((40, 1), np.int32)
    _check_align(ids, 5, 16)                  # experts 1..4 empty
    counts, offsets, sorted_ids, tile_expert, num_tiles = O.align_sort(np.zeros((0, 2), np.int32), 4, 16)
    assert counts.tolist() == [0] * 4 and num_tiles == 0 and len(sorted_ids) == 0


def test_align_capacity_bound_is_tight_when_every_expert_has_one_row():
    # E experts each with exactly one row pad to E*bm rows, which the bound allows
    E, bm = 8, 32
    ids = np.arange(E, dtype=np.int32).reshape(E, 1)
    counts, offsets, sorted_ids, tile_expert, num_tiles = O.align_sort(ids, E, bm)
    assert offsets[-1] == E * bm <= O.sorted_capacity(E, 1, E, bm)
