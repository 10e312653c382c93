"""ctypes binding of libmoe_mi355x.so (include/moe_mi355x.h).

Argument marshalling only: every step of the routed forward runs in the HIP
kernels behind the C ABI. torch supplies device memory (tensor.data_ptr())
and streams (torch.cuda.current_stream().cuda_stream). If the library is not
built, or no gfx950 GPU is current, every compute call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355x.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED_SHAPE = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_DEVICE = 4
MOE_NOALLOC_MAX_ASSIGNMENTS = 262144     # include/moe_mi355x.h: T * k limit of moe_align_sort_noalloc

DTYPE_BF16 = 0
DTYPE_FP8_BLOCK128 = 1
DTYPE_MXFP4W_MXFP8A = 2
ACT_SWIGLU = 0      # W1 [E, 2I, H] gate + up, h = silu(gate) * up
ACT_RELU2 = 1       # W1 [E, I, H], h = max(g, 0)^2
SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1

# name -> (restype, argtypes); mirrors include/moe_mi355x.h
_P, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "moe_route": (_I32, [_P, _I64, _I32, _I32, _I32, _P, _P, _P]),
    "moe_route_shared": (_I32, [_P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "moe_pick_block_m": (_I32, [_I32, _I64, _I32, _I32, _I32, _I32]),
    "moe_sorted_capacity": (_I64, [_I64, _I32, _I32, _I32]),
    "moe_align_sort_workspace_bytes": (_SZ, [_I64, _I32, _I32]),
    "moe_align_sort": (_I32, [_P, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_align_sort_noalloc": (_I32, [_P, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P]),
    "moe_quantize_fp8": (_I32, [_P, _I64, _I64, _I32, _P, _P, _P]),
    "moe_quantize_mxfp8": (_I32, [_P, _I64, _I64, _P, _P, _P]),
    "moe_quantize_mxfp4": (_I32, [_P, _I64, _I64, _P, _P, _P]),
    "moe_grouped_gemm_swiglu": (_I32, [_I32, _P, _P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32,
                                       _I32, _I64, _P, _P, _P, _SZ, _P]),
    "moe_grouped_gemm_workspace_bytes": (_SZ, []),
    "moe_grouped_gemm_swiglu_h32": (_I32, [_I32, _P, _P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32,
                                           _I32, _I64, _P, _P, _P, _P, _SZ, _P]),
    "moe_grouped_gemm_relu2": (_I32, [_I32, _P, _P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32,
                                      _I32, _I64, _P, _P, _P, _SZ, _P]),
    "moe_grouped_gemm_down": (_I32, [_I32, _P, _P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32,
                                     _I32, _I64, _P, _P, _SZ, _P]),
    "moe_combine": (_I32, [_P, _P, _I64, _I32, _I32, _P, _P]),
    "moe_down_combine_workspace_bytes": (_SZ, [_I64, _I32]),
    "moe_grouped_gemm_down_combine": (_I32, [_I32, _P, _P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32,
                                             _I32, _I64, _P, _P, _P, _P, _SZ, _P]),
    "moe_grouped_gemm_swiglu_save": (_I32, [_P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _I64,
                                            _P, _P, _P]),
    "moe_backward_combine": (_I32, [_P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I64, _P, _P, _P]),
    "moe_route_backward": (_I32, [_P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P, _P]),
    "moe_gather_rows": (_I32, [_P, _P, _P, _I64, _I32, _I32, _I32, _I64, _P, _P]),
    "moe_grouped_gemm_dh": (_I32, [_P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _I64, _P, _P]),
    "moe_grouped_gemm_dx": (_I32, [_P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _I64, _P, _P]),
    "moe_grouped_gemm_wgrad": (_I32, [_P, _P, _I32, _I32, _P, _I64, _I32, _I32, _I32, _I64, _P, _P]),
    "moe_status_string": (ctypes.c_char_p, [_I32]),
}

_lib = None


class MoeError(RuntimeError):
    def __init__(self, call: str, status: int):
        super().__init__(f"{call} failed: {moe_status_string(status)} ({status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the library once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python mixture_experts_routed_top_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(name: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(name, status)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _s(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, dtype, name: str, numel: Optional[int] = None, cols: Optional[int] = None):
    """Reject, before the C ABI sees it, an operand whose kernels would read or
    write past its end: the wrong dtype, device or layout, fewer than `numel`
    elements, or a last dimension other than `cols`."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a tensor, got {type(t).__name__}")
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous CUDA {dtype} tensor, got {t.dtype} on {t.device}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: needs at least {numel} elements, has {t.numel()} (shape {tuple(t.shape)})")
    if cols is not None and t.dim() > 0 and t.shape[-1] != cols:
        raise ValueError(f"{name}: last dimension must be {cols}, shape is {tuple(t.shape)}")


# element dtype of the token-side operands (x, h) and of the scales per numeric path
_VAL_DT = {DTYPE_BF16: torch.bfloat16, DTYPE_FP8_BLOCK128: torch.uint8, DTYPE_MXFP4W_MXFP8A: torch.uint8}
_SCALE = {DTYPE_FP8_BLOCK128: (torch.float32, 128), DTYPE_MXFP4W_MXFP8A: (torch.uint8, 32)}


def _check_gemm(dtype: int, gemm1: bool, gated: bool, a, a_scale, w, w_scale, sort: "SortResult", H: int, I: int,
                out, out_scale):
    """Sizes of every grouped-GEMM operand against the sort result and the
    layouts of include/moe_mi355x.h (a: x [T, H] or h [cap, I]; w: one row of
    K = H or I per output row of each expert; out: h [cap, I] or y [T*k, H])."""
    if dtype not in _VAL_DT:
        raise ValueError(f"unknown dtype {dtype}")
    T, k, E, cap = sort.T, sort.k, sort.E, sort.cap
    if T == 0:
        return
    K = H if gemm1 else I
    n_w = (2 * I if gated else I) if gemm1 else H          # weight rows of one expert
    rows_a = T if gemm1 else cap
    vdt = _VAL_DT[dtype]
    _need(a, vdt, "x" if gemm1 else "h", rows_a * K, K)
    if dtype == DTYPE_BF16:
        _need(w, torch.bfloat16, "w", E * n_w * K, K)
    else:
        sdt, g = _SCALE[dtype]
        if K % g or (gemm1 and I % g):
            return                                          # the C ABI reports the unsupported shape
        _need(a_scale, sdt, "x_scale" if gemm1 else "h_scale", rows_a * (K // g), K // g)
        if dtype == DTYPE_FP8_BLOCK128:
            _need(w, torch.uint8, "w", E * n_w * K, K)
            _need(w_scale, torch.float32, "w_scale", E * n_w // 128 * (K // 128), K // 128)
        else:
            _need(w, torch.uint8, "w", E * n_w * K // 2, K // 2)
            _need(w_scale, torch.uint8, "w_scale", E * n_w * (K // 32), K // 32)
    if gemm1:
        _need(out, vdt, "h", cap * I, I)
        if dtype != DTYPE_BF16:
            sdt, g = _SCALE[dtype]
            _need(out_scale, sdt, "h_scale", cap * (I // g), I // g)
    else:
        _need(out, torch.bfloat16, "y", T * k * H, H)


# ---------------------------------------------------------------- host-only queries
def moe_pick_block_m(dtype: int, T: int, k: int, E: int, H: int, I: int) -> int:
    return lib().moe_pick_block_m(dtype, T, k, E, H, I)


def moe_sorted_capacity(T: int, k: int, E: int, block_m: int) -> int:
    return lib().moe_sorted_capacity(T, k, E, block_m)


def moe_align_sort_workspace_bytes(T: int, k: int, E: int) -> int:
    return lib().moe_align_sort_workspace_bytes(T, k, E)


# ---------------------------------------------------------------- compute calls
def moe_route(logits: torch.Tensor, k: int, score: int = SCORE_SOFTMAX, topk_ids=None, topk_w=None,
              stream=None):
    _need(logits, torch.float32, "logits")
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _need(topk_ids, torch.int32, "topk_ids", T * k)
    _need(topk_w, torch.float32, "topk_w", T * k)
    _check("moe_route", lib().moe_route(_p(logits), T, E, k, score, _p(topk_ids), _p(topk_w), _s(stream)))
    return topk_ids, topk_w


def moe_route_shared(logits: torch.Tensor, k: int, score: int, n_shared: int, topk_ids=None, topk_w=None,
                     stream=None):
    _need(logits, torch.float32, "logits")
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty((T, k + n_shared), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, k + n_shared), dtype=torch.float32, device=logits.device)
    _need(topk_ids, torch.int32, "topk_ids", T * (k + n_shared))
    _need(topk_w, torch.float32, "topk_w", T * (k + n_shared))
    _check("moe_route_shared", lib().moe_route_shared(_p(logits), T, E, k, score, n_shared, _p(topk_ids),
                                                      _p(topk_w), _s(stream)))
    return topk_ids, topk_w


class SortResult:
    """Outputs of moe_align_sort (device tensors)."""

    def __init__(self, T, k, E, block_m, device):
        self.T, self.k, self.E, self.block_m = T, k, E, block_m
        self.cap = moe_sorted_capacity(T, k, E, block_m)
        self.counts = torch.empty(E, dtype=torch.int32, device=device)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=device)
        self.sorted_ids = torch.empty(max(self.cap, 1), dtype=torch.int32, device=device)
        self.tile_expert = torch.empty(max(self.cap // block_m, 1), dtype=torch.int32, device=device)
        self.num_tiles = torch.zeros(1, dtype=torch.int32, device=device)
        nbytes = moe_align_sort_workspace_bytes(T, k, E)
        self.ws = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=device)
        self.ws_bytes = nbytes


def moe_align_sort(topk_ids: torch.Tensor, E: int, block_m: int, out: Optional[SortResult] = None,
                   stream=None) -> SortResult:
    _need(topk_ids, torch.int32, "topk_ids")
    T, k = topk_ids.shape
    if out is None:
        out = SortResult(T, k, E, block_m, topk_ids.device)
    elif (out.T, out.k, out.E, out.block_m) != (T, k, E, block_m):
        raise ValueError(f"moe_align_sort: the SortResult was made for (T, k, E, block_m) = "
                         f"{(out.T, out.k, out.E, out.block_m)}, not {(T, k, E, block_m)}")
    _check("moe_align_sort", lib().moe_align_sort(
        _p(topk_ids), T, k, E, block_m, _p(out.counts), _p(out.offsets), _p(out.sorted_ids),
        _p(out.tile_expert), _p(out.num_tiles), _p(out.ws), out.ws_bytes, _s(stream)))
    return out


def moe_align_sort_noalloc(topk_ids: torch.Tensor, E: int, block_m: int, out: SortResult, stream=None) -> SortResult:
    """moe_align_sort with the library's fixed scratch instead of a workspace
    (no device allocation in the call; `out` must be prepared beforehand)."""
    _need(topk_ids, torch.int32, "topk_ids")
    T, k = topk_ids.shape
    if (out.T, out.k, out.E, out.block_m) != (T, k, E, block_m):
        raise ValueError("moe_align_sort_noalloc: the SortResult was made for another problem")
    _check("moe_align_sort_noalloc", lib().moe_align_sort_noalloc(
        _p(topk_ids), T, k, E, block_m, _p(out.counts), _p(out.offsets), _p(out.sorted_ids),
        _p(out.tile_expert), _p(out.num_tiles), _s(stream)))
    return out


def moe_quantize_fp8(x: torch.Tensor, block_rows: int = 1, q=None, scale=None, stream=None):
    _need(x, torch.bfloat16, "x")
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((rows // block_rows, cols // 128), dtype=torch.float32, device=x.device)
    _need(q, torch.uint8, "q", rows * cols)
    _need(scale, torch.float32, "scale", (rows // block_rows) * (cols // 128))
    _check("moe_quantize_fp8", lib().moe_quantize_fp8(_p(x), rows, cols, block_rows, _p(q), _p(scale),
                                                      _s(stream)))
    return q, scale


def moe_quantize_mxfp8(x: torch.Tensor, q=None, e8m0=None, stream=None):
    _need(x, torch.bfloat16, "x")
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if e8m0 is None:
        e8m0 = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    _need(q, torch.uint8, "q", rows * cols)
    _need(e8m0, torch.uint8, "e8m0", rows * (cols // 32))
    _check("moe_quantize_mxfp8", lib().moe_quantize_mxfp8(_p(x), rows, cols, _p(q), _p(e8m0), _s(stream)))
    return q, e8m0


def moe_quantize_mxfp4(x: torch.Tensor, q=None, e8m0=None, stream=None):
    _need(x, torch.bfloat16, "x")
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    if e8m0 is None:
        e8m0 = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    _need(q, torch.uint8, "q", rows * (cols // 2))
    _need(e8m0, torch.uint8, "e8m0", rows * (cols // 32))
    _check("moe_quantize_mxfp4", lib().moe_quantize_mxfp4(_p(x), rows, cols, _p(q), _p(e8m0), _s(stream)))
    return q, e8m0


def _h_alloc(dtype, cap, I, device):
    if dtype == DTYPE_BF16:
        return torch.empty((cap, I), dtype=torch.bfloat16, device=device), None
    h = torch.empty((cap, I), dtype=torch.uint8, device=device)
    if dtype == DTYPE_FP8_BLOCK128:
        return h, torch.empty((cap, I // 128), dtype=torch.float32, device=device)
    return h, torch.empty((cap, I // 32), dtype=torch.uint8, device=device)


def moe_grouped_gemm_workspace(device) -> torch.Tensor:
    """Workspace of the grouped GEMM calls on `device`, zero-filled (calls leave its counters zero)."""
    with torch.cuda.device(device):
        n = lib().moe_grouped_gemm_workspace_bytes()
    if n == 0:
        raise RuntimeError("moe_grouped_gemm_workspace_bytes: no supported device")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def _ws(ws):
    """(pointer, bytes) of an optional grouped-GEMM workspace."""
    if ws is None:
        return None, 0
    _need(ws, torch.uint8, "ws")
    return _p(ws), ws.numel()


def moe_grouped_gemm_swiglu(dtype: int, x, x_scale, w1, w1_scale, sort: SortResult, H: int, I: int,
                            h=None, h_scale=None, stream=None, ws=None):
    if h is None:
        h, h_scale = _h_alloc(dtype, max(sort.cap, 1), I, x.device)
    _check_gemm(dtype, True, True, x, x_scale, w1, w1_scale, sort, H, I, h, h_scale)
    _check("moe_grouped_gemm_swiglu", lib().moe_grouped_gemm_swiglu(
        dtype, _p(x), _p(x_scale), _p(w1), _p(w1_scale), _p(sort.sorted_ids), _p(sort.tile_expert),
        _p(sort.num_tiles), sort.T, H, I, sort.E, sort.k, sort.block_m, sort.cap, _p(h), _p(h_scale),
        *_ws(ws), _s(stream)))
    return h, h_scale


def moe_grouped_gemm_swiglu_h32(dtype: int, x, x_scale, w1, w1_scale, sort: SortResult, H: int, I: int,
                                h=None, h_scale=None, h32=None, stream=None, ws=None):
    """moe_grouped_gemm_swiglu that also returns the fp32 h before its storage
    rounding: (h, h_scale, h32 [cap, I] fp32)."""
    if h is None:
        h, h_scale = _h_alloc(dtype, max(sort.cap, 1), I, x.device)
    if h32 is None:
        h32 = torch.empty((max(sort.cap, 1), I), dtype=torch.float32, device=x.device)
    _check_gemm(dtype, True, True, x, x_scale, w1, w1_scale, sort, H, I, h, h_scale)
    _need(h32, torch.float32, "h32", sort.cap * I, I)
    _check("moe_grouped_gemm_swiglu_h32", lib().moe_grouped_gemm_swiglu_h32(
        dtype, _p(x), _p(x_scale), _p(w1), _p(w1_scale), _p(sort.sorted_ids), _p(sort.tile_expert),
        _p(sort.num_tiles), sort.T, H, I, sort.E, sort.k, sort.block_m, sort.cap, _p(h), _p(h_scale), _p(h32),
        *_ws(ws),
        _s(stream)))
    return h, h_scale, h32


def moe_grouped_gemm_relu2(dtype: int, x, x_scale, w1, w1_scale, sort: SortResult, H: int, I: int,
                           h=None, h_scale=None, stream=None, ws=None):
    if h is None:
        h, h_scale = _h_alloc(dtype, max(sort.cap, 1), I, x.device)
    _check_gemm(dtype, True, False, x, x_scale, w1, w1_scale, sort, H, I, h, h_scale)
    _check("moe_grouped_gemm_relu2", lib().moe_grouped_gemm_relu2(
        dtype, _p(x), _p(x_scale), _p(w1), _p(w1_scale), _p(sort.sorted_ids), _p(sort.tile_expert),
        _p(sort.num_tiles), sort.T, H, I, sort.E, sort.k, sort.block_m, sort.cap, _p(h), _p(h_scale),
        *_ws(ws), _s(stream)))
    return h, h_scale


def moe_grouped_gemm_down(dtype: int, h, h_scale, w2, w2_scale, sort: SortResult, H: int, I: int, y=None,
                          stream=None, ws=None):
    if y is None:
        y = torch.empty((max(sort.T * sort.k, 1), H), dtype=torch.bfloat16, device=h.device)
    _check_gemm(dtype, False, True, h, h_scale, w2, w2_scale, sort, H, I, y, None)
    _check("moe_grouped_gemm_down", lib().moe_grouped_gemm_down(
        dtype, _p(h), _p(h_scale), _p(w2), _p(w2_scale), _p(sort.sorted_ids), _p(sort.tile_expert),
        _p(sort.num_tiles), sort.T, H, I, sort.E, sort.k, sort.block_m, sort.cap, _p(y), *_ws(ws),
        _s(stream)))
    return y


def moe_down_combine_workspace(T: int, H: int, device) -> torch.Tensor:
    """Zeroed counter workspace of moe_grouped_gemm_down_combine (calls leave it zero)."""
    n = lib().moe_down_combine_workspace_bytes(T, H) // 4
    return torch.zeros(max(n, 1), dtype=torch.int32, device=device)


def moe_grouped_gemm_down_combine(dtype: int, h, h_scale, w2, w2_scale, sort: SortResult, H: int, I: int,
                                  topk_w, counters, y=None, out=None, stream=None):
    """GEMM2 with the weighted combine fused: returns (y, out)."""
    _need(topk_w, torch.float32, "topk_w")
    _need(counters, torch.int32, "counters")
    if y is None:
        y = torch.empty((max(sort.T * sort.k, 1), H), dtype=torch.bfloat16, device=h.device)
    if out is None:
        out = torch.empty((sort.T, H), dtype=torch.bfloat16, device=h.device)
    _check_gemm(dtype, False, True, h, h_scale, w2, w2_scale, sort, H, I, y, None)
    _need(topk_w, torch.float32, "topk_w", sort.T * sort.k)
    _need(out, torch.bfloat16, "out", sort.T * H, H)
    _check("moe_grouped_gemm_down_combine", lib().moe_grouped_gemm_down_combine(
        dtype, _p(h), _p(h_scale), _p(w2), _p(w2_scale), _p(sort.sorted_ids), _p(sort.tile_expert),
        _p(sort.num_tiles), sort.T, H, I, sort.E, sort.k, sort.block_m, sort.cap, _p(y), _p(topk_w), _p(out),
        _p(counters), counters.numel() * 4, _s(stream)))
    return y, out


def moe_combine(y: torch.Tensor, topk_w: torch.Tensor, out=None, stream=None):
    _need(y, torch.bfloat16, "y")
    _need(topk_w, torch.float32, "topk_w")
    T, k = topk_w.shape
    H = y.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _need(y, torch.bfloat16, "y", T * k * H, H)
    _need(out, torch.bfloat16, "out", T * H, H)
    _check("moe_combine", lib().moe_combine(_p(y), _p(topk_w), T, k, H, _p(out), _s(stream)))
    return out


# ---------------------------------------------------------------- backward (BF16)
def moe_grouped_gemm_swiglu_save(x, w1, sort: SortResult, H: int, I: int, h=None, gu=None, stream=None):
    """BF16 GEMM1 + SwiGLU that also stores the bf16 pre-activations gu [cap, 2I]."""
    if h is None:
        h = torch.empty((max(sort.cap, 1), I), dtype=torch.bfloat16, device=x.device)
    if gu is None:
        gu = torch.empty((max(sort.cap, 1), 2 * I), dtype=torch.bfloat16, device=x.device)
    _check_gemm(DTYPE_BF16, True, True, x, None, w1, None, sort, H, I, h, None)
    _need(gu, torch.bfloat16, "gu", sort.cap * 2 * I, 2 * I)
    _check("moe_grouped_gemm_swiglu_save", lib().moe_grouped_gemm_swiglu_save(
        _p(x), _p(w1), _p(sort.sorted_ids), _p(sort.tile_expert), _p(sort.num_tiles), sort.T, H, I, sort.E,
        sort.k, sort.block_m, sort.cap, _p(h), _p(gu), _s(stream)))
    return h, gu


def moe_backward_combine(dout, topk_w, y, sort: SortResult, dy=None, dw=None, stream=None):
    """dY [cap, H] bf16 (w * dout in sorted rows) and dw [T, k] fp32 (dout . y)."""
    _need(dout, torch.bfloat16, "dout")
    _need(topk_w, torch.float32, "topk_w")
    _need(y, torch.bfloat16, "y")
    T, k = topk_w.shape
    H = dout.shape[1]
    if dy is None:
        dy = torch.empty((max(sort.cap, 1), H), dtype=torch.bfloat16, device=dout.device)
    if dw is None:
        dw = torch.empty((T, k), dtype=torch.float32, device=dout.device)
    _need(dout, torch.bfloat16, "dout", T * H, H)
    _need(y, torch.bfloat16, "y", T * k * H, H)
    _need(dy, torch.bfloat16, "dy", sort.cap * H, H)
    _need(dw, torch.float32, "dw", T * k)
    _check("moe_backward_combine", lib().moe_backward_combine(
        _p(dout), _p(topk_w), _p(y), _p(sort.sorted_ids), _p(sort.num_tiles), T, k, H, sort.block_m, sort.cap,
        _p(dy), _p(dw), _s(stream)))
    return dy, dw


def moe_route_backward(topk_w, topk_ids, dw, E: int, k: int, score: int, n_shared: int = 0, dlogits=None,
                       stream=None):
    """dlogits [T, E] fp32 from the gate-weight gradient dw [T, k + n_shared]."""
    _need(topk_w, torch.float32, "topk_w")
    _need(topk_ids, torch.int32, "topk_ids")
    _need(dw, torch.float32, "dw")
    T = topk_w.shape[0]
    if dlogits is None:
        dlogits = torch.empty((T, E), dtype=torch.float32, device=dw.device)
    for name, t in (("topk_w", topk_w), ("topk_ids", topk_ids), ("dw", dw)):
        _need(t, t.dtype, name, T * (k + n_shared))
    _need(dlogits, torch.float32, "dlogits", T * E, E)
    _check("moe_route_backward", lib().moe_route_backward(
        _p(topk_w), _p(topk_ids), _p(dw), T, E, k, n_shared, score, _p(dlogits), _s(stream)))
    return dlogits


def moe_gather_rows(x, sort: SortResult, out=None, stream=None):
    """x in sorted-row order [cap, H] (pad rows 0)."""
    _need(x, torch.bfloat16, "x")
    H = x.shape[1]
    if out is None:
        out = torch.empty((max(sort.cap, 1), H), dtype=torch.bfloat16, device=x.device)
    _need(x, torch.bfloat16, "x", sort.T * H, H)
    _need(out, torch.bfloat16, "x_sorted", sort.cap * H, H)
    _check("moe_gather_rows", lib().moe_gather_rows(_p(x), _p(sort.sorted_ids), _p(sort.num_tiles), sort.T, sort.k,
                                                    H, sort.block_m, sort.cap, _p(out), _s(stream)))
    return out


def moe_grouped_gemm_dh(dy, w2, gu, sort: SortResult, H: int, I: int, dgu=None, stream=None):
    """dGU [cap, 2I] bf16: dY W2 through the SwiGLU backward."""
    if dgu is None:
        dgu = torch.empty((max(sort.cap, 1), 2 * I), dtype=torch.bfloat16, device=dy.device)
    _need(dy, torch.bfloat16, "dy", sort.cap * H, H)
    _need(w2, torch.bfloat16, "w2", sort.E * H * I, I)
    _need(gu, torch.bfloat16, "gu", sort.cap * 2 * I, 2 * I)
    _need(dgu, torch.bfloat16, "dgu", sort.cap * 2 * I, 2 * I)
    _check("moe_grouped_gemm_dh", lib().moe_grouped_gemm_dh(
        _p(dy), _p(w2), _p(gu), _p(sort.sorted_ids), _p(sort.tile_expert), _p(sort.num_tiles), sort.T, H, I,
        sort.E, sort.k, sort.block_m, sort.cap, _p(dgu), _s(stream)))
    return dgu


def moe_grouped_gemm_dx(dgu, w1, sort: SortResult, H: int, I: int, dx_rows=None, stream=None):
    """dx rows [T*k, H] bf16 in assignment order."""
    if dx_rows is None:
        dx_rows = torch.empty((max(sort.T * sort.k, 1), H), dtype=torch.bfloat16, device=dgu.device)
    _need(dgu, torch.bfloat16, "dgu", sort.cap * 2 * I, 2 * I)
    _need(w1, torch.bfloat16, "w1", sort.E * 2 * I * H, H)
    _need(dx_rows, torch.bfloat16, "dx_rows", sort.T * sort.k * H, H)
    _check("moe_grouped_gemm_dx", lib().moe_grouped_gemm_dx(
        _p(dgu), _p(w1), _p(sort.sorted_ids), _p(sort.tile_expert), _p(sort.num_tiles), sort.T, H, I,
        sort.E, sort.k, sort.block_m, sort.cap, _p(dx_rows), _s(stream)))
    return dx_rows


def moe_grouped_gemm_wgrad(p_rows, q_rows, sort: SortResult, dw=None, stream=None):
    """dW [E, N, M] fp32 = sum over each expert's sorted rows of q_rows^T p_rows."""
    _need(p_rows, torch.bfloat16, "p_rows")
    _need(q_rows, torch.bfloat16, "q_rows")
    M, N = p_rows.shape[1], q_rows.shape[1]
    if dw is None:
        dw = torch.empty((sort.E, N, M), dtype=torch.float32, device=p_rows.device)
    _need(p_rows, torch.bfloat16, "p_rows", sort.cap * M, M)
    _need(q_rows, torch.bfloat16, "q_rows", sort.cap * N, N)
    _need(dw, torch.float32, "dw", sort.E * N * M, M)
    _check("moe_grouped_gemm_wgrad", lib().moe_grouped_gemm_wgrad(
        _p(p_rows), _p(q_rows), M, N, _p(sort.offsets), sort.T, sort.E, sort.k, sort.block_m, sort.cap,
        _p(dw), _s(stream)))
    return dw
