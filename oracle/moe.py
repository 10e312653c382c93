"""The routed-expert MoE MLP forward, written out plainly in float64 numpy.

Test infrastructure only (see ``oracle/__init__.py``).

Pages cited (titles as published):
  [TS70]   TileScale PR #70, "SM90 FP8 distributed MegaMoE example"
  [FI5129] FlashInfer PR #5129, expert-sorted I/O for the cuTile BF16 fused MoE
  [FI6465] FlashInfer PR #6465, Hopper MXFP4 x FP8 MegaMoE tuning candidates
  [GCMOE]  "GC-MoE on SM120" (arXiv 2611.16219), Abstract
  [LIG]    Liger-Kernel PR #1463, "Specialize SM90 MoE communication and fix
           backward synchronization"

What the method computes (every page agrees; [TS70] Summary/Design, [FI5129]
Description, [FI6465] Benchmark configuration, [LIG] MoEBenchmark results): a
router picks k experts per token; each picked expert applies a gate/up
projection, SwiGLU and a down projection; the k expert outputs are summed
with the top-k weights. Implemented as: route -> expert-sorted padded
permutation -> grouped GEMM1 + SwiGLU -> grouped GEMM2 -> weighted combine.

Readings where the pages are silent:
  * top-k ties go to the lower expert index; slots are in descending score;
  * weights are softmax over the k selected logits (== softmax over all E,
    renormalised over the top k), or sigmoid(logit) without renormalisation;
  * W1 is [E, 2I, H]: gate rows [0, I), up rows [I, 2I); h = silu(gate) * up;
    with the squared-ReLU activation ([FI5129] Tests run SwiGLU and ReLU2;
    Measured, the Nemotron shape) the expert is not gated: W1 is [E, I, H]
    and h = max(g, 0)^2;
  * the top-k weights are applied in the combine, in slot order j = 0..k-1;
  * shared experts (folded into the compute in the GC-MoE Abstract; fused
    shared-expert execution in [TS70] Summary) are S further experts every
    token uses, after its k routed slots, with weight 1 and no gate: expert
    ids E..E+S-1 (W1/W2 carry them as their last S experts), slots k..k+S-1;
  * storage points: h is bf16 (BF16 path), FP8 E4M3 + fp32 1x128 scale along
    I (FP8 path) or E4M3 + E8M0 1x32 along I (MX path); Y and out are bf16.
Everything between two storage points is float64.
"""
from __future__ import annotations

import math

import numpy as np

from . import formats as F

SCORE_SOFTMAX = 0      # softmax over the selected logits (top-k renormalised)
SCORE_SIGMOID = 1      # sigmoid(logit), no renormalisation (top-1 gate)

DTYPE_BF16 = 0
DTYPE_FP8_BLOCK128 = 1
DTYPE_MXFP4W_MXFP8A = 2

ACT_SWIGLU = 0         # W1 [E, 2I, H] (gate, up); h = silu(gate) * up
ACT_RELU2 = 1          # W1 [E, I, H]; h = max(g, 0)^2


# ============================================================================ route
def route(logits: np.ndarray, k: int, score: int = SCORE_SOFTMAX):
    """Top-k routing. [TS70] Design, "Kernel 1: dispatch + L1 + SwiGLU" routes
    inside the first kernel; the weighting follows the tiny-config statement
    "softmax then top-k renormalized".

    logits: fp32 values [T, E] (any float dtype; compared as given).
    Returns ids int32 [T, k] (descending score, ties -> lower expert id) and
    w fp32 [T, k] (computed in float64, rounded RN to fp32).
    """
    logits = np.asarray(logits)
    T, E = logits.shape
    if not (1 <= k <= E):
        raise ValueError("route: need 1 <= k <= E")
    l64 = logits.astype(np.float64)
    # stable sort on the negated logit: equal logits keep ascending expert id
    order = np.argsort(-l64, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(l64, ids.astype(np.int64), axis=1)
    if score == SCORE_SOFTMAX:
        z = np.exp(sel - sel[:, :1])
        w = z / z.sum(axis=1, keepdims=True)
    elif score == SCORE_SIGMOID:
        w = 1.0 / (1.0 + np.exp(-sel))
    else:
        raise ValueError("route: unknown score function")
    return ids, F.round_fp32(w).astype(np.float32)


def route_with_shared(logits: np.ndarray, k: int, score: int, n_shared: int):
    """Routing plus S shared experts: the top-k slots of `route` over the E
    routed logits, then slots k..k+S-1 holding experts E..E+S-1 with weight 1.

    Returns ids int32 [T, k+S], w fp32 [T, k+S]."""
    ids, w = route(logits, k, score)
    T, E = np.asarray(logits).shape
    sid = np.broadcast_to(np.arange(E, E + n_shared, dtype=np.int32), (T, n_shared))
    return (np.concatenate([ids, sid], axis=1).astype(np.int32),
            np.concatenate([w, np.ones((T, n_shared), np.float32)], axis=1))


# ============================================================================ align / sort
def sorted_capacity(T: int, k: int, E: int, block_m: int) -> int:
    """Upper bound on the padded sorted row count, a multiple of block_m.

    Each non-empty expert pads its rows up to a multiple of block_m, adding at
    most block_m - 1 rows, and at most min(E, T*k) experts are non-empty.
    """
    A = T * k
    bound = A + min(E, A) * (block_m - 1)
    return -(-bound // block_m) * block_m


def align_sort(ids: np.ndarray, E: int, block_m: int):
    """Expert-sorted, tile-padded permutation of the assignments.

    [FI5129] Description: GEMM1 writes into the padded expert-sorted row space,
    GEMM2 reads it contiguously and scatters back to assignment order; padded
    rows feed only output rows that are dropped. [TS70] (first commit note):
    one flat list of m-tasks replaces the per-tile rescan of experts. [LIG]
    Summary: empty experts must not stall the schedule (they own no tiles).

    Assignment a = t*k + j (token t, slot j). Returns
      counts[E], offsets[E+1] (padded, exclusive), sorted_ids[cap]
      (assignment ids sorted by (expert, a), pad entries = T*k),
      tile_expert[cap // block_m] (expert of each tile, -1 past the last),
      num_tiles.
    """
    T, k = ids.shape
    A = T * k
    flat = ids.reshape(-1).astype(np.int64)
    if A and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("align_sort: expert id out of range")
    cap = sorted_capacity(T, k, E, block_m)
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    padded = -(-counts // block_m) * block_m
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    order = np.argsort(flat, kind="stable")          # by expert, then by a
    sorted_ids = np.full(cap, A, dtype=np.int64)
    start = 0
    for e in range(E):
        c = counts[e]
        sorted_ids[offsets[e]:offsets[e] + c] = order[start:start + c]
        start += c
    num_tiles = int(offsets[E] // block_m)
    tile_expert = np.full(cap // block_m, -1, dtype=np.int64)
    for e in range(E):
        tile_expert[offsets[e] // block_m:offsets[e + 1] // block_m] = e
    return (counts.astype(np.int32), offsets.astype(np.int32), sorted_ids.astype(np.int32),
            tile_expert.astype(np.int32), num_tiles)


# ============================================================================ quantizers
def quantize_fp8_block(v: np.ndarray, block_rows: int, block_cols: int = 128):
    """FP8 E4M3 with one fp32 scale per block_rows x block_cols block.

    [TS70] Design: FP8 E4M3 inputs and weights with FP32 per-128-element
    scales. Activations use 1x128 blocks, weights 128x128 blocks.
    Per block: amax = max|v|; s = RN_fp32(amax / 448), s = 1 when amax = 0;
    code = E4M3_RN_SAT(RN_fp32(v / s)).
    v: float64 values [R, C] with R % block_rows == 0 and C % block_cols == 0.
    Returns codes uint8 [R, C], scales fp32 [R / block_rows, C / block_cols].
    """
    v = np.asarray(v, dtype=np.float64)
    R, C = v.shape
    if R % block_rows or C % block_cols:
        raise ValueError("quantize_fp8_block: shape not a multiple of the block")
    blocks = v.reshape(R // block_rows, block_rows, C // block_cols, block_cols)
    amax = np.abs(blocks).max(axis=(1, 3))
    s = F.round_fp32(amax / F.E4M3_MAX)
    s = np.where(amax == 0, 1.0, s)
    q = F.round_fp32(blocks / s[:, None, :, None])
    codes = F.e4m3_encode(q).reshape(R, C)
    return codes, s.astype(np.float32)


def dequantize_fp8_block(codes, scales, block_rows: int, block_cols: int = 128) -> np.ndarray:
    vals = F.e4m3_decode(codes)
    s = np.repeat(np.repeat(np.asarray(scales, np.float64), block_rows, axis=0), block_cols, axis=1)
    return vals * s


def _mx_shared_exponent(blocks: np.ndarray, emax_elem: int) -> np.ndarray:
    """OCP MX v1.0: X = 2^(floor(log2 amax) - emax_elem), exponent clamped to [-127, 127].

    Returns the E8M0 byte (exponent + 127); an all-zero block gives byte 0.
    """
    amax = np.abs(blocks).max(axis=-1)
    e = np.where(amax > 0, np.frexp(np.where(amax > 0, amax, 1.0))[1].astype(np.int64) - 1, -127)
    x = np.where(amax > 0, np.clip(e - emax_elem, -127, 127), -127)
    return (x + 127).astype(np.uint8)


def quantize_mxfp8(v: np.ndarray):
    """MXFP8 along the last axis: E4M3 elements, one E8M0 scale per 32.

    [FI6465] Benchmark configuration: FP8 activations against MXFP4 K32
    weights; the activations take the same 1x32 E8M0 block form (reading:
    the MX block-scaled matrix op takes E8M0 scales on both operands, as in
    [GCMOE] Abstract). Rule: OCP MX v1.0 (floor of log2 amax, emax_elem = 8).
    v: [R, C], C % 32 == 0. Returns codes uint8 [R, C], e8m0 uint8 [R, C/32].
    """
    v = np.asarray(v, dtype=np.float64)
    R, C = v.shape
    if C % 32:
        raise ValueError("quantize_mxfp8: columns must be a multiple of 32")
    blocks = v.reshape(R, C // 32, 32)
    sb = _mx_shared_exponent(blocks, 8)
    x = np.ldexp(1.0, sb.astype(np.int64) - 127)
    codes = F.e4m3_encode(blocks / x[..., None]).reshape(R, C)   # division by 2^n is exact
    return codes, sb


def quantize_mxfp4(v: np.ndarray):
    """MXFP4 along the last axis: E2M1 elements, one E8M0 scale per 32.

    [FI6465] Benchmark configuration (E2M1 weights, one shared scale per 32 along K).
    Rule: OCP MX v1.0 (emax_elem = 2). Two codes per byte, even column in the
    low nibble. v: [R, C], C % 32 == 0.
    Returns packed uint8 [R, C/2], e8m0 uint8 [R, C/32].
    """
    v = np.asarray(v, dtype=np.float64)
    R, C = v.shape
    if C % 32:
        raise ValueError("quantize_mxfp4: columns must be a multiple of 32")
    blocks = v.reshape(R, C // 32, 32)
    sb = _mx_shared_exponent(blocks, 2)
    x = np.ldexp(1.0, sb.astype(np.int64) - 127)
    codes = F.e2m1_encode(blocks / x[..., None]).reshape(R, C)
    return F.pack_e2m1(codes), sb


def dequantize_mxfp8(codes, e8m0) -> np.ndarray:
    vals = F.e4m3_decode(codes)
    return vals * np.repeat(F.e8m0_decode(e8m0), 32, axis=-1)


def dequantize_mxfp4(packed, e8m0) -> np.ndarray:
    vals = F.e2m1_decode(F.unpack_e2m1(packed))
    return vals * np.repeat(F.e8m0_decode(e8m0), 32, axis=-1)


# ============================================================================ expert MLP
def silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


def relu2(g: np.ndarray) -> np.ndarray:
    return np.square(np.maximum(g, 0.0))


def _activate(xa: np.ndarray, w1e: np.ndarray, act: int) -> np.ndarray:
    """The expert's first projection and activation for rows xa.

    SwiGLU: w1e [2I, H], gate rows first. ReLU2: w1e [I, H], no gate."""
    if act == ACT_SWIGLU:
        I = w1e.shape[0] // 2
        return silu(xa @ w1e[:I].T) * (xa @ w1e[I:].T)
    if act == ACT_RELU2:
        return relu2(xa @ w1e.T)
    raise ValueError("unknown activation")


def intermediate_size(w1_rows: int, act: int) -> int:
    """I from the row count of one expert's W1."""
    return w1_rows // 2 if act == ACT_SWIGLU else w1_rows


def _store_h(h: np.ndarray, dtype: int):
    """Storage point of the intermediate (reading listed in the module docstring).

    Returns (stored representation, its float64 value)."""
    if dtype == DTYPE_BF16:
        hb = F.round_bf16(h)
        return (hb, None), hb
    if dtype == DTYPE_FP8_BLOCK128:
        codes, s = quantize_fp8_block(h, 1, 128)
        return (codes, s), dequantize_fp8_block(codes, s, 1, 128)
    if dtype == DTYPE_MXFP4W_MXFP8A:
        codes, sb = quantize_mxfp8(h)
        return (codes, sb), dequantize_mxfp8(codes, sb)
    raise ValueError("unknown dtype")


def grouped_gemm_swiglu(x_hat: np.ndarray, w1_hat: np.ndarray, sorted_ids: np.ndarray,
                        tile_expert: np.ndarray, num_tiles: int, block_m: int, k: int,
                        dtype: int, act: int = ACT_SWIGLU):
    """GEMM1 + activation over the sorted rows, then the h storage point.

    [TS70] Design, Kernel 1 (L1 GEMM + SwiGLU, quantised intermediate);
    [FI5129] Description (GEMM1 writes padded expert-sorted rows) and Tests
    (SwiGLU and ReLU2).
    x_hat [T, H] and w1_hat [E, 2I, H] (SwiGLU) or [E, I, H] (ReLU2) are the
    (dequantised) float64 operands. Sorted row r (r < num_tiles * block_m)
    holding assignment a < T*k reads token a // k; pad rows read a zero row,
    so their h is 0.
    Returns (stored h, float64 value of stored h), both with num_tiles*block_m rows.
    """
    E, w1_rows, H = w1_hat.shape
    I = intermediate_size(w1_rows, act)
    A = x_hat.shape[0] * k
    rows = num_tiles * block_m
    h = np.zeros((rows, I), dtype=np.float64)
    for tile in range(num_tiles):
        e = int(tile_expert[tile])
        r0 = tile * block_m
        a = sorted_ids[r0:r0 + block_m].astype(np.int64)
        valid = a < A
        xa = np.zeros((block_m, H), dtype=np.float64)
        xa[valid] = x_hat[a[valid] // k]
        h[r0:r0 + block_m] = _activate(xa, w1_hat[e], act)
    return _store_h(h, dtype)


def grouped_gemm_down(h_val: np.ndarray, w2_hat: np.ndarray, sorted_ids: np.ndarray,
                      tile_expert: np.ndarray, num_tiles: int, block_m: int, A: int):
    """GEMM2 over the sorted rows; each real row lands in assignment order.

    [FI5129] Description: GEMM2 reads A contiguously from the sorted rows and
    its epilogue scatters to assignment order; pad rows are dropped.
    [TS70] Design, Kernel 2: rows land per (token, top-k slot).
    h_val [rows, I] float64, w2_hat [E, H, I]. Returns Y float64 (bf16
    values) [A, H].
    """
    E, H, I = w2_hat.shape
    y = np.zeros((A, H), dtype=np.float64)
    for tile in range(num_tiles):
        e = int(tile_expert[tile])
        r0 = tile * block_m
        a = sorted_ids[r0:r0 + block_m].astype(np.int64)
        valid = a < A
        yt = h_val[r0:r0 + block_m] @ w2_hat[e].T
        y[a[valid]] = F.round_bf16(yt[valid])
    return y


def combine(y: np.ndarray, w: np.ndarray) -> np.ndarray:
    """out[t] = bf16( sum_j w[t, j] * Y[t*k + j] ), summed in float64.

    [TS70] review thread "reduce tail" (the reduce over top-k slots to a BF16
    output) and [FI5129] Description (the combine follows GEMM2 unchanged).
    """
    T, k = w.shape
    H = y.shape[1]
    acc = np.zeros((T, H), dtype=np.float64)
    for j in range(k):
        acc += np.asarray(w[:, j], np.float64)[:, None] * y[j::k]
    return F.round_bf16(acc)


# ============================================================================ whole forward
def moe_forward(logits, x_bf16, w1_bf16, w2_bf16, k: int, score: int, dtype: int,
                block_m: int = 16, w1_q=None, w2_q=None, act: int = ACT_SWIGLU, n_shared: int = 0):
    """The whole routed forward for one batch.

    x_bf16 [T, H], w1_bf16 [E, 2I, H] (SwiGLU) or [E, I, H] (ReLU2),
    w2_bf16 [E, H, I]: float64 arrays of bf16 values; with n_shared = S > 0
    the last S experts of w1/w2 are shared (logits cover the E - S routed ones). For the FP8 path x is
    quantised 1x128 and the weights 128x128 (w1_q / w2_q may pass precomputed
    (codes, scales)); for the MX path x is MXFP8 1x32 and the weights MXFP4
    1x32 along K.
    Returns a dict of every intermediate.
    """
    x_bf16 = np.asarray(x_bf16, np.float64)
    T, H = x_bf16.shape
    E, twoI, _ = w1_bf16.shape     # twoI: rows of one expert's W1 (2I, or I for ReLU2)
    I = intermediate_size(twoI, act)
    if n_shared:
        ids, w = route_with_shared(logits, k, score, n_shared)
        k = k + n_shared
    else:
        ids, w = route(logits, k, score)
    counts, offsets, sorted_ids, tile_expert, num_tiles = align_sort(ids, E, block_m)
    out = {"ids": ids, "w": w, "counts": counts, "offsets": offsets,
           "sorted_ids": sorted_ids, "tile_expert": tile_expert, "num_tiles": num_tiles}
    if dtype == DTYPE_BF16:
        x_hat = x_bf16
        w1_hat = np.asarray(w1_bf16, np.float64)
        w2_hat = np.asarray(w2_bf16, np.float64)
    elif dtype == DTYPE_FP8_BLOCK128:
        xq, xs = quantize_fp8_block(x_bf16, 1, 128)
        x_hat = dequantize_fp8_block(xq, xs, 1, 128)
        if w1_q is None:
            w1_q = quantize_fp8_block(np.asarray(w1_bf16).reshape(E * twoI, H), 128, 128)
        if w2_q is None:
            w2_q = quantize_fp8_block(np.asarray(w2_bf16).reshape(E * H, I), 128, 128)
        w1_hat = dequantize_fp8_block(*w1_q, 128, 128).reshape(E, twoI, H)
        w2_hat = dequantize_fp8_block(*w2_q, 128, 128).reshape(E, H, I)
        out.update(xq=xq, xs=xs)
    elif dtype == DTYPE_MXFP4W_MXFP8A:
        xq, xs = quantize_mxfp8(x_bf16)
        x_hat = dequantize_mxfp8(xq, xs)
        if w1_q is None:
            w1_q = quantize_mxfp4(np.asarray(w1_bf16).reshape(E * twoI, H))
        if w2_q is None:
            w2_q = quantize_mxfp4(np.asarray(w2_bf16).reshape(E * H, I))
        w1_hat = dequantize_mxfp4(*w1_q).reshape(E, twoI, H)
        w2_hat = dequantize_mxfp4(*w2_q).reshape(E, H, I)
        out.update(xq=xq, xs=xs)
    else:
        raise ValueError("unknown dtype")
    (h_store, h_val) = grouped_gemm_swiglu(x_hat, w1_hat, sorted_ids, tile_expert, num_tiles,
                                           block_m, k, dtype, act)
    y = grouped_gemm_down(h_val, w2_hat, sorted_ids, tile_expert, num_tiles, block_m, T * k)
    out.update(h=h_store, h_val=h_val, y=y, out=combine(y, w))
    return out


def routed_flops(T: int, k: int, H: int, I: int, act: int = ACT_SWIGLU) -> int:
    """Routed FLOPs of one forward: the two grouped GEMMs, 6*T*k*H*I for
    SwiGLU (GEMM1 has 2I outputs per row), 4*T*k*H*I for the ungated ReLU2.

    [LIG] MoEBenchmark results: shared experts and attention are not counted;
    the router projection, the activation and combine are not GEMM work either.
    """
    return (6 if act == ACT_SWIGLU else 4) * T * k * H * I


def assignment_forward(x_row, w1e, w2e, dtype: int = DTYPE_BF16, act: int = ACT_SWIGLU):
    """One (token, expert) row of Y computed on its own: the same arithmetic as
    grouped_gemm_swiglu + grouped_gemm_down restricted to one assignment.

    x_row [H] dequantised token, w1e [2I, H] (or [I, H] for ReLU2) and w2e
    [H, I] the expert's dequantised weights. Returns float64 bf16 values [H]."""
    hv_raw = _activate(np.asarray(x_row, np.float64)[None, :], np.asarray(w1e, np.float64), act)
    _, hv = _store_h(hv_raw, dtype)
    return F.round_bf16(np.asarray(w2e, np.float64) @ hv[0])


def token_forward(x_row, w1_hat, w2_hat, ids_row, w_row, dtype: int = DTYPE_BF16, act: int = ACT_SWIGLU):
    """One token's output computed on its own (used for sampled checks at
    full size: same arithmetic as moe_forward restricted to one token).

    x_row [H] dequantised input, ids_row/w_row [k]. Returns float64 bf16 values [H].
    """
    acc = np.zeros(np.asarray(w2_hat[int(ids_row[0])]).shape[0], dtype=np.float64)
    for j, e in enumerate(ids_row):   # w1_hat / w2_hat: arrays [E, ...] or dicts of experts
        acc += float(w_row[j]) * assignment_forward(x_row, w1_hat[e], w2_hat[e], dtype, act)
    return F.round_bf16(acc)


__all__ = [n for n in dir() if not n.startswith("_") and n not in ("math", "np", "F")]


# ============================================================================ backward
# The backward of the BF16 SwiGLU routed forward, for a given output gradient
# dout (training). Readings where the pages are silent: the top-k selection is
# piecewise constant (no gradient through the choice); the forward saves the
# gate/up pre-activations in bf16 beside h; storage points of the backward:
# dY and dGU (the operands of the next GEMMs) and the per-assignment dx rows
# are bf16, dx is bf16, the weight gradients and dw / dlogits are fp32.
def route_backward(w: np.ndarray, ids: np.ndarray, dw: np.ndarray, E: int, score: int) -> np.ndarray:
    """dlogits [T, E] from the gradient dw [T, k] of the routed weights.

    SOFTMAX over the selected logits: dl_i = w_i (dw_i - sum_j w_j dw_j) for
    selected i; SIGMOID: dl_i = dw_i w_i (1 - w_i). Unselected logits: 0."""
    w = np.asarray(w, np.float64)
    dw = np.asarray(dw, np.float64)
    T, k = w.shape
    if score == SCORE_SOFTMAX:
        g = w * (dw - (w * dw).sum(axis=1, keepdims=True))
    else:
        g = dw * w * (1.0 - w)
    dl = np.zeros((T, E), dtype=np.float64)
    np.put_along_axis(dl, np.asarray(ids, np.int64), g, axis=1)
    return F.round_fp32(dl).astype(np.float32)


def _row_layout(sorted_ids, tile_expert, num_tiles: int, block_m: int, A: int):
    """Sorted rows r < num_tiles * block_m: assignment ids, real-row mask and
    the expert of each row."""
    rows = num_tiles * block_m
    srt = np.asarray(sorted_ids[:rows], np.int64)
    real = srt < A
    e_of = np.repeat(np.asarray(tile_expert[:num_tiles], np.int64), block_m)
    return rows, srt, real, e_of


def _per_expert(e_of, E: int, rows: int, out_cols: int, f):
    """Rows of expert e (e_of == e) filled by f(e, sel); other rows 0."""
    out = np.zeros((rows, out_cols))
    for e in range(E):
        sel = e_of == e
        if sel.any():
            out[sel] = f(e, sel)
    return out


def gate_up_rows(x, w1, sorted_ids, tile_expert, num_tiles: int, block_m: int, kk: int):
    """GEMM1 of the backward's saved forward, per sorted row: the token row x[a // kk]
    (0 for pad rows) against its expert's gate rows W1[e, :I] and up rows
    W1[e, I:]. Returns (xs, g, u): the gathered rows and both projections, float64."""
    x = np.asarray(x, np.float64)
    w1 = np.asarray(w1, np.float64)
    E, twoI, _ = w1.shape
    I = twoI // 2
    rows, srt, real, e_of = _row_layout(sorted_ids, tile_expert, num_tiles, block_m, x.shape[0] * kk)
    tok = np.where(real, srt // kk, 0)
    xs = np.where(real[:, None], x[tok], 0.0)                       # gathered tokens, sorted rows
    g = _per_expert(e_of, E, rows, I, lambda e, sel: xs[sel] @ w1[e, :I].T)
    u = _per_expert(e_of, E, rows, I, lambda e, sel: xs[sel] @ w1[e, I:].T)
    return xs, g, u


def combine_backward(dout, w, y, sorted_ids, num_tiles: int, block_m: int, exact: bool = False):
    """Backward of the weighted combine out[t] = sum_j w[t, j] y[t*kk + j]:
    dY of each sorted row, dy[r] = bf16(w[a] * dout[a // kk]) (0 for pad rows),
    and the gate-weight gradient dw[t, j] = sum_c dout[t, c] y[t*kk + j, c] (float64).
    w: [T, kk]; y: [T*kk, H] in assignment order."""
    rb = (lambda v: np.asarray(v, np.float64)) if exact else F.round_bf16
    dout = np.asarray(dout, np.float64)
    y = np.asarray(y, np.float64)
    T, kk = np.asarray(w).shape
    A = T * kk
    rows = num_tiles * block_m
    srt = np.asarray(sorted_ids[:rows], np.int64)
    real = srt < A
    tok = np.where(real, srt // kk, 0)
    wa = np.asarray(w, np.float64).reshape(A)
    dy = np.where(real[:, None], rb(wa[np.where(real, srt, 0)][:, None] * dout[tok]), 0.0)
    dw = (dout[np.arange(A) // kk] * y).sum(axis=1).reshape(T, kk)
    return dy, dw


def swiglu_backward(dy, w2, gu, tile_expert, num_tiles: int, block_m: int, exact: bool = False):
    """Gradient through GEMM2 and the SwiGLU, per sorted row of expert e:
    dh = dy @ W2[e] (float64); with (g, u) the saved pre-activations gu[r]
    and s = sigmoid(g): dgu = bf16([dh u s (1 + g (1 - s)), dh g s])."""
    rb = (lambda v: np.asarray(v, np.float64)) if exact else F.round_bf16
    dy = np.asarray(dy, np.float64)
    w2 = np.asarray(w2, np.float64)
    gu = np.asarray(gu, np.float64)
    E, H, I = w2.shape
    rows = num_tiles * block_m
    e_of = np.repeat(np.asarray(tile_expert[:num_tiles], np.int64), block_m)
    g_s, u_s = gu[:rows, :I], gu[:rows, I:]
    dh = _per_expert(e_of, E, rows, I, lambda e, sel: dy[sel] @ w2[e])
    sg = 1.0 / (1.0 + np.exp(-g_s))
    dg = dh * u_s * sg * (1.0 + g_s * (1.0 - sg))
    du = dh * g_s * sg
    return rb(np.concatenate([dg, du], axis=1))


def dx_rows_backward(dgu, w1, sorted_ids, tile_expert, num_tiles: int, block_m: int, A: int,
                     exact: bool = False):
    """Gradient through GEMM1 to each assignment's row: dx_rows[a] =
    bf16(dgu[r] @ W1[e]) for the sorted row r of assignment a, in assignment
    order [A, H]."""
    rb = (lambda v: np.asarray(v, np.float64)) if exact else F.round_bf16
    dgu = np.asarray(dgu, np.float64)
    w1 = np.asarray(w1, np.float64)
    E, _, H = w1.shape
    rows, srt, real, e_of = _row_layout(sorted_ids, tile_expert, num_tiles, block_m, A)
    dx_sorted = rb(_per_expert(e_of, E, rows, H, lambda e, sel: dgu[sel] @ w1[e]))
    dx_rows = np.zeros((A, H))
    dx_rows[srt[real]] = dx_sorted[real]
    return dx_rows


def weight_grad(p_rows, q_rows, sorted_ids, tile_expert, num_tiles: int, block_m: int, A: int, E: int):
    """Per-expert weight gradient over the expert's real sorted rows:
    dW[e] = sum_r q_rows[r]^T p_rows[r] (float64) [E, N, M]; dW2 takes
    p = h, q = dy; dW1 takes p = the gathered token rows, q = dgu."""
    p_rows = np.asarray(p_rows, np.float64)
    q_rows = np.asarray(q_rows, np.float64)
    rows, srt, real, e_of = _row_layout(sorted_ids, tile_expert, num_tiles, block_m, A)
    dw = np.zeros((E, q_rows.shape[1], p_rows.shape[1]))
    for e in range(E):
        sel = (e_of == e) & real
        if sel.any():
            dw[e] = q_rows[:rows][sel].T @ p_rows[:rows][sel]
    return dw


def moe_backward(logits, x_bf16, w1_bf16, w2_bf16, dout_bf16, k: int, score: int, block_m: int = 16,
                 n_shared: int = 0, exact: bool = False):
    """Gradients of the BF16 SwiGLU routed forward (moe_forward) for dout.

    Returns a dict: dx [T, H], dw1 [E, 2I, H], dw2 [E, H, I], dw [T, k(+S)],
    dlogits [T, E_routed], and the stored intermediates dy (sorted rows),
    dgu (sorted rows), dx_rows (assignment order). exact=True drops every
    storage rounding (forward and backward), which makes the result the
    mathematical gradient of the unrounded forward.
    """
    rb = (lambda v: np.asarray(v, np.float64)) if exact else F.round_bf16
    x = np.asarray(x_bf16, np.float64)
    w1 = np.asarray(w1_bf16, np.float64)
    w2 = np.asarray(w2_bf16, np.float64)
    dout = np.asarray(dout_bf16, np.float64)
    T, H = x.shape
    E, twoI, _ = w1.shape
    E_routed = E - n_shared
    if n_shared:
        ids, w = route_with_shared(logits, k, score, n_shared)
    else:
        ids, w = route(logits, k, score)
    kk = k + n_shared
    A = T * kk
    counts, offsets, sorted_ids, tile_expert, num_tiles = align_sort(ids, E, block_m)
    rows, srt, real, e_of = _row_layout(sorted_ids, tile_expert, num_tiles, block_m, A)

    # forward, saving what the backward reads
    xs, g, u = gate_up_rows(x, w1, sorted_ids, tile_expert, num_tiles, block_m, kk)
    h = rb(silu(g) * u)
    y_sorted = rb(_per_expert(e_of, E, rows, H, lambda e, sel: h[sel] @ w2[e].T))
    y = np.zeros((A, H))
    y[srt[real]] = y_sorted[real]
    gu = np.concatenate([rb(g), rb(u)], axis=1)                     # saved pre-activations

    # combine backward, router backward
    dy, dw = combine_backward(dout, w, y, sorted_ids, num_tiles, block_m, exact)
    dw32 = F.round_fp32(dw).astype(np.float32)
    dlogits = route_backward(w[:, :k], ids[:, :k], dw[:, :k], E_routed, score)
    # GEMM2 backward through the SwiGLU; the weight gradients; GEMM1 backward
    # to the dx rows, then the sum over each token's slots
    dgu = swiglu_backward(dy, w2, gu, tile_expert, num_tiles, block_m, exact)
    dw2 = weight_grad(h, dy, sorted_ids, tile_expert, num_tiles, block_m, A, E)
    dw1 = weight_grad(xs, dgu, sorted_ids, tile_expert, num_tiles, block_m, A, E)
    dx_rows = dx_rows_backward(dgu, w1, sorted_ids, tile_expert, num_tiles, block_m, A, exact)
    dx = rb(dx_rows.reshape(T, kk, H).sum(axis=1))
    f32 = (lambda v: v) if exact else (lambda v: F.round_fp32(v))
    return {"ids": ids, "w": w, "sorted_ids": sorted_ids, "tile_expert": tile_expert, "num_tiles": num_tiles,
            "gu": gu, "h": h, "y": y,
            "dy": dy, "dw": dw32, "dlogits": dlogits, "dgu": dgu, "dx_rows": dx_rows, "dx": dx,
            "dw1": f32(dw1), "dw2": f32(dw2)}
