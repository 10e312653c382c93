"""The routed forward as one object: weights prepared once, buffers planned
per token count, then route -> align_sort -> [quantise x] -> GEMM1+activation ->
GEMM2 -> combine on one stream with no allocation and no host sync.

For the BF16 SwiGLU layer, forward_train / backward run one training step
over the same sorted layout: the forward also keeps the pre-activations, and
the backward chains combine-backward -> router-backward -> dGU -> dx rows ->
dx, and the two weight gradients.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import _binding as B


@dataclass
class Plan:
    T: int
    block_m: int
    ids: torch.Tensor
    w: torch.Tensor
    sort: B.SortResult
    xq: Optional[torch.Tensor]
    xs: Optional[torch.Tensor]
    h: torch.Tensor
    h_scale: Optional[torch.Tensor]
    y: torch.Tensor
    out: torch.Tensor
    train: Optional["TrainBuffers"] = None
    counters: Optional[torch.Tensor] = None      # fused combine: zeroed counter workspace
    ws: Optional[torch.Tensor] = None            # BF16 GEMMs: zeroed K-split workspace (last-round balance)


@dataclass
class TrainBuffers:
    """What the backward reads from the forward, and the gradient outputs."""
    gu: torch.Tensor          # [cap, 2I] bf16 pre-activations
    dy: torch.Tensor          # [cap, H] bf16
    dw: torch.Tensor          # [T, k] fp32 gate-weight gradient
    dlogits: torch.Tensor     # [T, E_routed] fp32
    dgu: torch.Tensor         # [cap, 2I] bf16
    dx_rows: torch.Tensor     # [T*k, H] bf16
    dx: torch.Tensor          # [T, H] bf16
    x_sorted: torch.Tensor    # [cap, H] bf16
    ones: torch.Tensor        # [T, k] fp32, unit weights of the dx reduction
    dw1: torch.Tensor         # [E, 2I, H] fp32
    dw2: torch.Tensor         # [E, H, I] fp32


class MoeLayer:
    """Routed-expert MoE MLP forward on one GPU.

    w1: [E, 2I, H] bf16 (gate rows [0, I), up rows [I, 2I)), or [E, I, H] for
    the ungated squared-ReLU expert (act=ACT_RELU2, BF16 only); w2: [E, H, I] bf16.
    With n_shared = S > 0 the last S experts of w1/w2 are shared experts that
    every token uses with weight 1 (the router scores the first E - S only);
    they run in the same sorted layout and task queue as the routed ones.
    For the FP8 path the weights are quantised here to E4M3 with 128x128 fp32
    block scales, for the MX path to E2M1 with E8M0 per 32 along K (weight
    preparation, outside the timed forward).

    fused_combine=True (BF16) runs GEMM2 with the weighted combine in its
    epilogue (same result, bit for bit, but slower on MI355X: the device-scope
    fences between the workgroups of different XCDs flush the L2 weight reuse).
    plan(T, train=True) prepares the BF16 SwiGLU training step:
    forward_train() keeps the pre-activations and backward() returns dx,
    dlogits and the fp32 weight gradients dw1, dw2.
    """

    def __init__(self, dtype: int, w1: torch.Tensor, w2: torch.Tensor, k: int, score: int = B.SCORE_SOFTMAX,
                 act: int = B.ACT_SWIGLU, n_shared: int = 0, fused_combine: bool = False,
                 split_tail: bool = True):
        E, twoI, H = w1.shape
        if act not in (B.ACT_SWIGLU, B.ACT_RELU2):
            raise ValueError("unknown activation")
        if act == B.ACT_RELU2 and dtype != B.DTYPE_BF16:
            raise ValueError("the squared-ReLU expert is BF16 only")
        if fused_combine and dtype != B.DTYPE_BF16:
            raise ValueError("the fused combine is implemented for the BF16 path")
        self.dtype, self.score, self.act, self.n_shared = dtype, score, act, n_shared
        self.fused_combine = fused_combine
        # the BF16 GEMMs split their last round of tiles along K when given a workspace
        self.split_tail = split_tail and dtype == B.DTYPE_BF16
        self.k_routed, self.k = k, k + n_shared          # slots per token: routed, then shared
        self.E, self.H, self.I = E, H, (twoI // 2 if act == B.ACT_SWIGLU else twoI)
        if w2.shape != (E, H, self.I):
            raise ValueError("w2 must be [E, H, I]")
        self.w1_scale = self.w2_scale = None
        if dtype == B.DTYPE_BF16:
            self.w1, self.w2 = w1.contiguous(), w2.contiguous()
        elif dtype == B.DTYPE_FP8_BLOCK128:
            self.w1, self.w1_scale = B.moe_quantize_fp8(w1.reshape(E * twoI, H).contiguous(), 128)
            self.w2, self.w2_scale = B.moe_quantize_fp8(w2.reshape(E * H, self.I).contiguous(), 128)
        elif dtype == B.DTYPE_MXFP4W_MXFP8A:
            self.w1, self.w1_scale = B.moe_quantize_mxfp4(w1.reshape(E * twoI, H).contiguous())
            self.w2, self.w2_scale = B.moe_quantize_mxfp4(w2.reshape(E * H, self.I).contiguous())
        else:
            raise ValueError("unknown dtype")

    def plan(self, T: int, block_m: Optional[int] = None, device=None, train: bool = False) -> Plan:
        device = device or self.w1.device
        if train:
            if self.dtype != B.DTYPE_BF16 or self.act != B.ACT_SWIGLU:
                raise ValueError("the training step is implemented for the BF16 SwiGLU layer")
            block_m = 256                                  # the backward GEMMs' row tile
        bm = block_m or B.moe_pick_block_m(self.dtype, T, self.k, self.E, self.H, self.I)
        sort = B.SortResult(T, self.k, self.E, bm, device)
        xq = xs = None
        if self.dtype == B.DTYPE_FP8_BLOCK128:
            xq = torch.empty((T, self.H), dtype=torch.uint8, device=device)
            xs = torch.empty((T, self.H // 128), dtype=torch.float32, device=device)
        elif self.dtype == B.DTYPE_MXFP4W_MXFP8A:
            xq = torch.empty((T, self.H), dtype=torch.uint8, device=device)
            xs = torch.empty((T, self.H // 32), dtype=torch.uint8, device=device)
        h, h_scale = B._h_alloc(self.dtype, max(sort.cap, 1), self.I, device)
        tb = None
        if train:
            cap, A, H, I, E = max(sort.cap, 1), max(T * self.k, 1), self.H, self.I, self.E
            bf, f32 = torch.bfloat16, torch.float32
            tb = TrainBuffers(
                gu=torch.empty((cap, 2 * I), dtype=bf, device=device),
                dy=torch.empty((cap, H), dtype=bf, device=device),
                dw=torch.empty((T, self.k), dtype=f32, device=device),
                dlogits=torch.empty((T, E - self.n_shared), dtype=f32, device=device),
                dgu=torch.empty((cap, 2 * I), dtype=bf, device=device),
                dx_rows=torch.empty((A, H), dtype=bf, device=device),
                dx=torch.empty((T, H), dtype=bf, device=device),
                x_sorted=torch.empty((cap, H), dtype=bf, device=device),
                ones=torch.ones((T, self.k), dtype=f32, device=device),
                dw1=torch.empty((E, 2 * I, H), dtype=f32, device=device),
                dw2=torch.empty((E, H, I), dtype=f32, device=device))
        return Plan(T, bm,
                    torch.empty((T, self.k), dtype=torch.int32, device=device),
                    torch.empty((T, self.k), dtype=torch.float32, device=device),
                    sort, xq, xs, h, h_scale,
                    torch.empty((max(T * self.k, 1), self.H), dtype=torch.bfloat16, device=device),
                    torch.empty((T, self.H), dtype=torch.bfloat16, device=device), tb,
                    B.moe_down_combine_workspace(T, self.H, device) if self.fused_combine else None,
                    B.moe_grouped_gemm_workspace(device) if self.split_tail and T > 0 else None)

    def forward(self, x: torch.Tensor, logits: torch.Tensor, plan: Optional[Plan] = None,
                stream=None) -> torch.Tensor:
        T = x.shape[0]
        p = plan if plan is not None else self.plan(T, device=x.device)
        if p.T != T:
            raise ValueError("plan was made for another token count")
        self._route(logits, p, stream)
        B.moe_align_sort(p.ids, self.E, p.block_m, out=p.sort, stream=stream)
        if self.dtype == B.DTYPE_BF16:
            a, a_scale = x, None
        elif self.dtype == B.DTYPE_FP8_BLOCK128:
            a, a_scale = B.moe_quantize_fp8(x, 1, p.xq, p.xs, stream=stream)
        else:
            a, a_scale = B.moe_quantize_mxfp8(x, p.xq, p.xs, stream=stream)
        gemm1 = B.moe_grouped_gemm_swiglu if self.act == B.ACT_SWIGLU else B.moe_grouped_gemm_relu2
        gemm1(self.dtype, a, a_scale, self.w1, self.w1_scale, p.sort, self.H, self.I, p.h, p.h_scale,
              stream=stream, ws=p.ws)
        if self.fused_combine:
            B.moe_grouped_gemm_down_combine(self.dtype, p.h, p.h_scale, self.w2, self.w2_scale, p.sort, self.H,
                                            self.I, p.w, p.counters, p.y, p.out, stream=stream)
            return p.out
        B.moe_grouped_gemm_down(self.dtype, p.h, p.h_scale, self.w2, self.w2_scale, p.sort, self.H, self.I,
                                p.y, stream=stream, ws=p.ws)
        return B.moe_combine(p.y, p.w, p.out, stream=stream)

    __call__ = forward

    def _route(self, logits, p: Plan, stream):
        if self.n_shared:
            B.moe_route_shared(logits, self.k_routed, self.score, self.n_shared, p.ids, p.w, stream=stream)
        else:
            B.moe_route(logits, self.k, self.score, p.ids, p.w, stream=stream)

    def forward_train(self, x: torch.Tensor, logits: torch.Tensor, plan: Plan, stream=None) -> torch.Tensor:
        """The BF16 SwiGLU forward that keeps what backward needs (plan made with train=True)."""
        if plan.train is None or plan.T != x.shape[0]:
            raise ValueError("forward_train needs a training plan for this token count")
        p = plan
        self._route(logits, p, stream)
        B.moe_align_sort(p.ids, self.E, p.block_m, out=p.sort, stream=stream)
        B.moe_grouped_gemm_swiglu_save(x, self.w1, p.sort, self.H, self.I, p.h, p.train.gu, stream=stream)
        B.moe_grouped_gemm_down(self.dtype, p.h, None, self.w2, None, p.sort, self.H, self.I, p.y, stream=stream,
                                ws=p.ws)
        return B.moe_combine(p.y, p.w, p.out, stream=stream)

    def backward(self, x: torch.Tensor, dout: torch.Tensor, plan: Plan, stream=None) -> TrainBuffers:
        """Gradients for dout of the last forward_train with this plan: dx, dlogits, dw1, dw2 (fp32)."""
        p, tb = plan, plan.train
        if tb is None:
            raise ValueError("backward needs a training plan")
        H, I = self.H, self.I
        B.moe_backward_combine(dout, p.w, p.y, p.sort, tb.dy, tb.dw, stream=stream)
        B.moe_route_backward(p.w, p.ids, tb.dw, self.E - self.n_shared, self.k_routed, self.score, self.n_shared,
                             tb.dlogits, stream=stream)
        B.moe_grouped_gemm_dh(tb.dy, self.w2, tb.gu, p.sort, H, I, tb.dgu, stream=stream)
        B.moe_grouped_gemm_dx(tb.dgu, self.w1, p.sort, H, I, tb.dx_rows, stream=stream)
        B.moe_combine(tb.dx_rows, tb.ones, tb.dx, stream=stream)
        B.moe_gather_rows(x, p.sort, tb.x_sorted, stream=stream)
        B.moe_grouped_gemm_wgrad(p.h, tb.dy, p.sort, tb.dw2, stream=stream)
        B.moe_grouped_gemm_wgrad(tb.x_sorted, tb.dgu, p.sort, tb.dw1, stream=stream)
        return tb
