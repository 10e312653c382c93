"""C ABI checks that need no GPU: the library loads, exports every function
include/moe_mi355x.h declares, and rejects bad arguments on the host before
touching a device. No call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

from oracle import moe as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")

M = pytest.importorskip("mixture_experts_routed_top_amd")


def _lib():
    try:
        return M.lib()
    except RuntimeError as e:  # not built
        pytest.fail(str(e))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_0-9]+)\s*\(", text, flags=re.M)


def test_header_declares_the_boundary():
    names = set(declared_functions())
    for n in ["moe_route", "moe_align_sort", "moe_grouped_gemm_swiglu", "moe_grouped_gemm_down",
              "moe_combine", "moe_quantize_fp8", "moe_quantize_mxfp8", "moe_quantize_mxfp4",
              "moe_sorted_capacity", "moe_align_sort_workspace_bytes", "moe_pick_block_m",
              "moe_status_string", "moe_grouped_gemm_swiglu_save", "moe_backward_combine", "moe_route_backward",
              "moe_gather_rows", "moe_grouped_gemm_dh", "moe_grouped_gemm_dx", "moe_grouped_gemm_wgrad"]:
        assert n in names, n


def test_library_exports_every_declared_symbol():
    L = _lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    # the binding declares the same set with signatures
    assert set(declared_functions()) == set(M._binding.SIGNATURES)


def test_status_strings():
    assert M.moe_status_string(0) == "MOE_OK"
    assert M.moe_status_string(3) == "MOE_ERR_WORKSPACE"
    assert M.moe_status_string(99) == "MOE_ERR_UNKNOWN"


@pytest.mark.parametrize("T,k,E,bm", [(0, 2, 8, 16), (1, 1, 1, 16), (64, 2, 8, 32), (8192, 8, 128, 128),
                                      (16384, 10, 512, 16), (129, 10, 512, 64)])
def test_capacity_matches_oracle(T, k, E, bm):
    assert M.moe_sorted_capacity(T, k, E, bm) == O.sorted_capacity(T, k, E, bm)


def test_capacity_and_block_m_rejections():
    assert M.moe_sorted_capacity(10, 2, 8, 48) == -1
    assert M.moe_sorted_capacity(-1, 2, 8, 16) == -1
    assert M.moe_pick_block_m(0, 10, 9, 8, 256, 128) == -1          # k > E
    for dt in (0, 1, 2):
        for T in (1, 64, 1024, 8192, 16384):
            assert M.moe_pick_block_m(dt, T, 8, 128, 2048, 768) in (16, 32, 64, 128, 256)


# The row-tile rule at the named shapes' token counts (mean rows per expert in
# brackets), as measured with the current kernels: BF16 Qwen3-30B-A3B shape,
# FP8 64-expert H 7168 shape (256-row tiles from 384 rows, since its 64- and
# 128-row tiles split their LDS stages and the 256-row GEMM1 cannot), MXFP4
# 512-expert shape.
@pytest.mark.parametrize("dt,T,k,E,H,I,bm", [
    (0, 512, 8, 128, 2048, 768, 64), (0, 2048, 8, 128, 2048, 768, 128), (0, 8192, 8, 128, 2048, 768, 256),
    (1, 256, 8, 64, 7168, 2048, 64), (1, 512, 8, 64, 7168, 2048, 128), (1, 2048, 8, 64, 7168, 2048, 128),
    (1, 4096, 8, 64, 7168, 2048, 256), (1, 8192, 8, 64, 7168, 2048, 256),
    (2, 128, 10, 512, 2560, 640, 32), (2, 2048, 10, 512, 2560, 640, 64), (2, 16384, 10, 512, 2560, 640, 128)])
def test_pick_block_m_rule(dt, T, k, E, H, I, bm):
    assert M.moe_pick_block_m(dt, T, k, E, H, I) == bm


def test_workspace_bytes():
    assert M.moe_align_sort_workspace_bytes(0, 8, 128) == 0
    assert M.moe_align_sort_workspace_bytes(64, 2, 8) == 4 * (1 * 8 + 128)
    assert M.moe_align_sort_workspace_bytes(8192, 8, 128) == 4 * (64 * 128 + 65536)


NULL = None
FAKE = 0x10000  # 16-byte aligned non-null address; never dereferenced by these calls
MIS = 0x10002   # misaligned


def test_route_host_validation():
    L = _lib()
    assert L.moe_route(FAKE, 4, 8, 9, 0, FAKE, FAKE, NULL) == M._binding.MOE_ERR_INVALID_ARG  # k > E
    assert L.moe_route(FAKE, 4, 8, 0, 0, FAKE, FAKE, NULL) == 1
    assert L.moe_route(FAKE, 4, 2000, 2, 0, FAKE, FAKE, NULL) == 1                           # E too large
    assert L.moe_route(FAKE, 4, 8, 2, 7, FAKE, FAKE, NULL) == 1                              # score
    assert L.moe_route(NULL, 4, 8, 2, 0, FAKE, FAKE, NULL) == 1
    assert L.moe_route(MIS, 4, 8, 2, 0, FAKE, FAKE, NULL) == 1
    assert L.moe_route(NULL, 0, 8, 2, 0, NULL, NULL, NULL) == 0                              # T = 0
    assert L.moe_route(FAKE, -1, 8, 2, 0, FAKE, FAKE, NULL) == 1
    assert L.moe_route_shared(FAKE, 4, 8, 2, 0, -1, FAKE, FAKE, NULL) == 1                    # n_shared < 0
    assert L.moe_route_shared(FAKE, 4, 64, 30, 0, 3, FAKE, FAKE, NULL) == 1                   # k + S > 32
    assert L.moe_route_shared(FAKE, 4, 1024, 2, 0, 1, FAKE, FAKE, NULL) == 1                  # E + S > 1024
    assert L.moe_route_shared(NULL, 0, 8, 2, 0, 1, NULL, NULL, NULL) == 0


def test_align_sort_host_validation():
    L = _lib()
    ws = M.moe_align_sort_workspace_bytes(64, 2, 8)
    args = lambda bm, wsb, ids=FAKE: (ids, 64, 2, 8, bm, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wsb, NULL)
    assert L.moe_align_sort(*args(48, ws)) == 1
    assert L.moe_align_sort(*args(16, ws - 4)) == M._binding.MOE_ERR_WORKSPACE
    assert L.moe_align_sort(*args(16, ws, NULL)) == 1
    assert L.moe_align_sort(NULL, 0, 2, 8, 16, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == 0


def test_quantize_host_validation():
    L = _lib()
    assert L.moe_quantize_fp8(FAKE, 128, 100, 1, FAKE, FAKE, NULL) == M._binding.MOE_ERR_UNSUPPORTED_SHAPE
    assert L.moe_quantize_fp8(FAKE, 100, 128, 128, FAKE, FAKE, NULL) == 2
    assert L.moe_quantize_fp8(FAKE, 128, 128, 64, FAKE, FAKE, NULL) == 1
    assert L.moe_quantize_fp8(MIS, 128, 128, 1, FAKE, FAKE, NULL) == 1
    assert L.moe_quantize_mxfp8(FAKE, 4, 40, FAKE, FAKE, NULL) == 2
    assert L.moe_quantize_mxfp4(FAKE, 4, 40, FAKE, FAKE, NULL) == 2
    assert L.moe_quantize_mxfp4(NULL, 0, 64, NULL, NULL, NULL) == 0


def _gemm_args(dtype=0, T=64, H=256, I=128, E=8, k=2, bm=32, cap=None, x=FAKE, w=FAKE, out=FAKE):
    cap = O.sorted_capacity(T, k, E, bm) if cap is None else cap
    return (dtype, x, FAKE, w, FAKE, FAKE, FAKE, FAKE, T, H, I, E, k, bm, cap)


def test_gemm_host_validation():
    L = _lib()
    sw = lambda *a, **kw: L.moe_grouped_gemm_swiglu(*_gemm_args(*a, **kw), FAKE, FAKE, NULL, 0, NULL)
    r2 = lambda *a, **kw: L.moe_grouped_gemm_relu2(*_gemm_args(*a, **kw), FAKE, FAKE, NULL, 0, NULL)
    dn = lambda *a, **kw: L.moe_grouped_gemm_down(*_gemm_args(*a, **kw), FAKE, NULL, 0, NULL)
    # the squared-ReLU GEMM1 is BF16 only, rejected before anything is enqueued
    assert r2(dtype=1, H=256, I=128) == 2
    assert r2(dtype=2, H=256, I=128, T=0, x=NULL, w=NULL) == 2
    for f in (sw, r2, dn):
        assert f(dtype=5) == 1
        assert f(H=100) == 2                    # bf16 needs H % 8 == 0
        assert f(dtype=1, H=192) == 2           # fp8 needs H % 128 == 0
        assert f(dtype=2, I=96) == 2            # mx needs I % 128 == 0
        assert f(bm=48) == 1
        assert f(cap=12345) == 1                # capacity must be the queried one
        assert f(k=9) == 1
        assert f(x=NULL) == 1
        assert f(w=MIS) == 1
        assert f(T=0, x=NULL, w=NULL) == 0
    # the optional K-split workspace must be 256-byte aligned (checked before the device)
    assert L.moe_grouped_gemm_swiglu(*_gemm_args(), FAKE, FAKE, MIS, 1 << 30, NULL) == 1
    assert L.moe_grouped_gemm_relu2(*_gemm_args(), FAKE, FAKE, MIS, 1 << 30, NULL) == 1
    assert L.moe_grouped_gemm_down(*_gemm_args(), FAKE, MIS, 1 << 30, NULL) == 1


def test_combine_host_validation():
    L = _lib()
    assert L.moe_combine(FAKE, FAKE, 4, 2, 100, FAKE, NULL) == 2
    assert L.moe_combine(FAKE, FAKE, 4, 0, 128, FAKE, NULL) == 1
    assert L.moe_combine(MIS, FAKE, 4, 2, 128, FAKE, NULL) == 1
    assert L.moe_combine(NULL, NULL, 0, 2, 128, NULL, NULL) == 0


def test_backward_host_validation():
    L = _lib()
    T, k, E, H, I = 64, 2, 4, 128, 64
    cap = O.sorted_capacity(T, k, E, 256)
    dh = lambda T=T, H=H, I=I, bm=256, cap=cap, dy=FAKE, gu=FAKE: L.moe_grouped_gemm_dh(
        dy, FAKE, gu, FAKE, FAKE, FAKE, T, H, I, E, k, bm, cap, FAKE, NULL)
    dx = lambda T=T, H=H, I=I, bm=256, cap=cap, dgu=FAKE: L.moe_grouped_gemm_dx(
        dgu, FAKE, FAKE, FAKE, FAKE, T, H, I, E, k, bm, cap, FAKE, NULL)
    wg = lambda M=I, N=H, bm=256, cap=cap, p=FAKE, dw=FAKE: L.moe_grouped_gemm_wgrad(
        p, FAKE, M, N, FAKE, T, E, k, bm, cap, dw, NULL)
    for f in (dh, dx):
        assert f(H=100) == 2                     # H % 8
        assert f(I=60) == 2                      # I % 8
        assert f(bm=64, cap=O.sorted_capacity(T, k, E, 64)) == 2   # the backward GEMMs tile 256 rows
        assert f(bm=48) == 1
        assert f(cap=cap + 256) == 1
        assert f(T=0, cap=0) == 0
    assert dh(dy=NULL) == 1 and dh(gu=MIS) == 1 and dx(dgu=MIS) == 1
    assert L.moe_grouped_gemm_dh(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, T, H, I, 2, 3, 256,
                                 O.sorted_capacity(T, 3, 2, 256), FAKE, NULL) == 1     # k > E
    assert wg(M=100) == 2 and wg(N=36) == 2 and wg(M=0) == 1
    assert wg(bm=128, cap=O.sorted_capacity(T, k, E, 128)) == 2
    assert wg(p=NULL) == 1 and wg(dw=MIS) == 1
    save = lambda h=FAKE, gu=FAKE, T=T, cap=cap: L.moe_grouped_gemm_swiglu_save(
        FAKE, FAKE, FAKE, FAKE, FAKE, T, H, I, E, k, 256, cap, h, gu, NULL)
    assert save(gu=NULL) == 1 and save(gu=MIS) == 1 and save(T=0, cap=0, gu=NULL) == 0
    bc = lambda y=FAKE, nt=FAKE, T=T, H=H, bm=256: L.moe_backward_combine(FAKE, FAKE, y, FAKE, nt, T, k, H, bm, cap,
                                                                          FAKE, FAKE, NULL)
    assert bc(H=100) == 2 and bc(y=MIS) == 1 and bc(nt=NULL) == 1 and bc(bm=48) == 1
    assert L.moe_backward_combine(NULL, NULL, NULL, NULL, NULL, 0, k, H, 256, cap, NULL, NULL, NULL) == 0
    assert L.moe_route_backward(FAKE, FAKE, FAKE, T, E, 5, 0, 0, FAKE, NULL) == 1     # k > E
    assert L.moe_route_backward(FAKE, FAKE, FAKE, T, E, 2, 0, 7, FAKE, NULL) == 1     # unknown score
    assert L.moe_route_backward(FAKE, FAKE, NULL, T, E, 2, 0, 0, FAKE, NULL) == 1
    assert L.moe_gather_rows(FAKE, FAKE, FAKE, T, k, 100, 256, cap, FAKE, NULL) == 2
    assert L.moe_gather_rows(FAKE, FAKE, FAKE, T, k, H, 256, cap, MIS, NULL) == 1
    assert L.moe_gather_rows(FAKE, FAKE, NULL, T, k, H, 256, cap, FAKE, NULL) == 1


def test_down_combine_host_validation():
    L = _lib()
    T, k, E, H, I, bm = 64, 2, 4, 256, 128, 32
    cap = O.sorted_capacity(T, k, E, bm)
    need = L.moe_down_combine_workspace_bytes(T, H)
    assert need == T * 2 * 4 and L.moe_down_combine_workspace_bytes(-1, H) == 0
    f = lambda dtype=0, ws=FAKE, nbytes=need, out=FAKE, T=T, cap=cap: L.moe_grouped_gemm_down_combine(
        dtype, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, T, H, I, E, k, bm, cap, FAKE, FAKE, out, ws, nbytes, NULL)
    assert f(dtype=1) == 2 and f(dtype=2) == 2          # BF16 only
    assert f(nbytes=need - 4) == 3                      # workspace below the size
    assert f(ws=NULL) == 1 and f(out=MIS) == 1
    assert f(T=0, cap=0) == 0


def test_device_check_without_gpu():
    # valid arguments reach the device check; without a gfx950 device current
    # the call must fail with MOE_ERR_DEVICE and launch nothing
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: fake pointers would be dereferenced")
    L = _lib()
    assert L.moe_route(FAKE, 4, 8, 2, 0, FAKE, FAKE, NULL) == M._binding.MOE_ERR_DEVICE


def test_compute_calls_reject_host_tensors():
    """Every compute call takes device tensors only: a host tensor is rejected
    with ValueError before the library is called, so nothing ever falls back
    to a CPU computation."""
    import torch
    logits = torch.zeros((4, 8), dtype=torch.float32)
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        M.moe_route(logits, 2)
    with pytest.raises(ValueError):
        M.moe_route_shared(logits, 2, 0, 1)
    with pytest.raises(ValueError):
        M.moe_align_sort(torch.zeros((4, 2), dtype=torch.int32), 8, 32)
    with pytest.raises(ValueError):
        M.moe_quantize_fp8(x, 1)
    with pytest.raises(ValueError):
        M.moe_quantize_mxfp8(x)
    with pytest.raises(ValueError):
        M.moe_quantize_mxfp4(x)
    with pytest.raises(ValueError):
        M.moe_combine(torch.zeros((8, 256), dtype=torch.bfloat16), torch.zeros((4, 2), dtype=torch.float32))
