"""GEMM2 with the weighted combine fused into its epilogue, through the C
ABI: its combined output must equal, bit for bit, the separate GEMM2 ->
combine path on the same inputs (both sum the k bf16 rows in fp32 in slot
order), and match the oracle's forward; the counter workspace must be zero
again after every call."""
import numpy as np
import pytest
import torch

import mixture_experts_routed_top_amd as M
from oracle import moe as O
from workloads import get_config, make_inputs, to_f64
from tests.gpu_util import TOL_COS, TOL_FRO, cuda, f64, min_row_cos, rel_fro, say

pytestmark = pytest.mark.gpu


def _both(cfg, inp, block_m=None, calls=2):
    layer = M.MoeLayer(M.DTYPE_BF16, cuda(inp.w1), cuda(inp.w2), cfg.k, cfg.score, n_shared=cfg.n_shared)
    plan = layer.plan(cfg.T, block_m=block_m)
    ref_out = layer(cuda(inp.x), cuda(inp.logits), plan).clone()
    ref_y = plan.y.clone()
    ws = M.moe_down_combine_workspace(cfg.T, cfg.H, "cuda:0")
    outs = []
    for _ in range(calls):
        y = torch.full_like(plan.y, 7)
        _, out = M.moe_grouped_gemm_down_combine(M.DTYPE_BF16, plan.h, None, layer.w2, None, plan.sort, cfg.H,
                                                 cfg.I, plan.w, ws, y=y)
        torch.cuda.synchronize()
        assert not ws.any(), "the counters must be left zero"
        assert torch.equal(y, ref_y)
        outs.append(out)
    return plan, ref_out, outs


@pytest.mark.parametrize("T,H,E,k,I,bm", [
    (200, 256, 8, 2, 128, None), (333, 640, 6, 3, 256, 32), (129, 384, 16, 4, 256, 64),
    (700, 1024, 16, 8, 512, 128), (900, 520, 4, 2, 256, 256), (1, 256, 8, 2, 128, None),
    (100, 256, 1, 1, 128, None),
])
def test_fused_combine_equals_separate(T, H, E, k, I, bm):
    cfg = get_config("tiny_bf16").with_(T=T, H=H, E=E, k=k, I=I, w_std=0.05)
    inp = make_inputs(cfg, seed=T + H)
    say("fused combine", T, H, E, k, I, bm)
    plan, ref_out, outs = _both(cfg, inp, bm)
    for out in outs:
        assert torch.equal(out, ref_out)
    ref = O.moe_forward(inp.logits.numpy(), to_f64(inp.x), to_f64(inp.w1), to_f64(inp.w2), cfg.k, cfg.score,
                        O.DTYPE_BF16, block_m=plan.block_m)
    got = f64(outs[0])
    assert rel_fro(got, ref["out"]) <= TOL_FRO[0]
    assert min_row_cos(got, ref["out"]) >= TOL_COS


def test_fused_combine_shared_expert():
    cfg = get_config("tiny_bf16").with_(T=150, H=256, E=6, k=2, I=128, n_shared=1, w_std=0.05)
    inp = make_inputs(cfg, seed=5)
    say("fused combine shared")
    _, ref_out, outs = _both(cfg, inp)
    assert torch.equal(outs[0], ref_out)


def test_fused_combine_full_size():
    """The Qwen3-30B-A3B-shaped workload at T = 8192 in the benchmark's launch
    configuration (the separate path is checked against the oracle by the
    forward tests)."""
    cfg = get_config("qwen3_30b_a3b_bf16")
    inp = make_inputs(cfg)
    say("fused combine full", cfg.name)
    _, ref_out, outs = _both(cfg, inp, calls=3)
    for out in outs:
        assert torch.equal(out, ref_out)


def test_layer_fused_combine_option():
    cfg = get_config("tiny_bf16").with_(T=300, E=8, k=2)
    inp = make_inputs(cfg, seed=2)
    say("layer fused combine")
    a = M.MoeLayer(M.DTYPE_BF16, cuda(inp.w1), cuda(inp.w2), cfg.k, cfg.score)
    b = M.MoeLayer(M.DTYPE_BF16, cuda(inp.w1), cuda(inp.w2), cfg.k, cfg.score, fused_combine=True)
    x, lg = cuda(inp.x), cuda(inp.logits)
    pa, pb = a.plan(cfg.T), b.plan(cfg.T)
    ra = a(x, lg, pa).clone()
    for _ in range(2):
        assert torch.equal(b(x, lg, pb), ra)
