"""moe_align_sort_noalloc (the allocation-free align_sort, fixed scratch)
through the C ABI: its outputs equal moe_align_sort's (workspace from the
caller) and the oracle's, bit for bit, on calls in a row, each with a smaller
problem that reuses the scratch the one before left behind."""
import numpy as np
import pytest
import torch

import mixture_experts_routed_top_amd as M
from oracle import moe as O
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _ids(T, E, k, seed):
    logits = np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32)
    return O.route(logits, k)[0]


def _filled(sort: M.SortResult, value: int) -> M.SortResult:
    for t in (sort.counts, sort.offsets, sort.sorted_ids, sort.tile_expert, sort.num_tiles):
        t.fill_(value)
    return sort


def test_align_sort_noalloc_matches_workspace_call():
    # each problem is smaller in T, k and E than the one before and uses another row tile;
    # the last (1600 assignments) takes the one-workgroup sort
    for T, E, k, bm, seed in [(16384, 512, 10, 64, 1), (700, 64, 4, 32, 2), (200, 32, 8, 16, 3)]:
        ids = _ids(T, E, k, seed)
        dids = torch.from_numpy(ids).to(DEV)
        say("align_sort_noalloc", T, E, k, bm)
        ref = M.moe_align_sort(dids, E, bm, out=_filled(M.SortResult(T, k, E, bm, DEV), -7))
        got = M.moe_align_sort_noalloc(dids, E, bm, out=_filled(M.SortResult(T, k, E, bm, DEV), -9))
        torch.cuda.synchronize()
        for name in ("counts", "offsets", "sorted_ids", "tile_expert", "num_tiles"):
            assert torch.equal(getattr(got, name), getattr(ref, name)), name
        counts, offsets, sorted_ids, tile_expert, num_tiles = O.align_sort(ids, E, bm)
        np.testing.assert_array_equal(got.counts.cpu().numpy(), counts)
        np.testing.assert_array_equal(got.offsets.cpu().numpy(), offsets)
        np.testing.assert_array_equal(got.sorted_ids.cpu().numpy()[:len(sorted_ids)], sorted_ids)
        np.testing.assert_array_equal(got.tile_expert.cpu().numpy()[:len(tile_expert)], tile_expert)
        assert int(got.num_tiles.item()) == num_tiles


def test_align_sort_noalloc_rejects_beyond_its_scratch():
    L = M.lib()
    ids = torch.zeros((1, 1), dtype=torch.int32, device=DEV)
    out = M.SortResult(1, 1, 4, 32, DEV)
    T = M._binding.MOE_NOALLOC_MAX_ASSIGNMENTS // 8 + 1          # T * k one tile past the limit
    st = L.moe_align_sort_noalloc(ids.data_ptr(), T, 8, 64, 32, out.counts.data_ptr(), out.offsets.data_ptr(),
                                  out.sorted_ids.data_ptr(), out.tile_expert.data_ptr(), out.num_tiles.data_ptr(),
                                  None)
    assert st == M._binding.MOE_ERR_WORKSPACE
