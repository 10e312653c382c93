"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the algorithmic
bytes behind the HBM roofline, and the rocprofv3 summary writer."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import get_config  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "4"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_bf16():
    cfg = get_config("qwen3_30b_a3b_bf16")
    A = cfg.T * cfg.k
    b1, _ = bench.gemm_algorithmic_bytes(cfg, "gemm1_swiglu", cfg.E)
    assert b1 == cfg.E * 2 * cfg.I * cfg.H * 2 + cfg.T * cfg.H * 2 + A * cfg.I * 2
    b2, _ = bench.gemm_algorithmic_bytes(cfg, "gemm2_down", 100)
    assert b2 == 100 * cfg.H * cfg.I * 2 + A * cfg.I * 2 + A * cfg.H * 2


def test_algorithmic_bytes_block_scaled():
    # MX: half a byte per E2M1 weight, one E8M0 byte per 32 elements on both operands
    cfg = get_config("mxfp4_moe_t128")
    A = cfg.T * cfg.k
    b1, _ = bench.gemm_algorithmic_bytes(cfg, "gemm1_swiglu", 7)
    w = 7 * 2 * cfg.I * cfg.H * (0.5 + 1 / 32)
    assert b1 == int(w + cfg.T * cfg.H * (1 + 1 / 32) + A * cfg.I * (1 + 1 / 32))
    # FP8: one fp32 per 128x128 weight block and per 1x128 token block
    cfg = get_config("fp8_block128_share")
    b2, _ = bench.gemm_algorithmic_bytes(cfg, "gemm2_down", cfg.E)
    A = cfg.T * cfg.k
    w = cfg.E * cfg.H * cfg.I * (1 + 4 / (128 * 128))
    assert b2 == int(w + A * cfg.I * (1 + 4 / 128) + A * cfg.H * 2)


def test_small_token_counts_are_hbm_bound():
    # the weights of every expert used dominate at T = 128: HBM time > MFMA time
    cfg = get_config("mxfp4_moe_t128")
    flops = 4 * cfg.T * cfg.k * cfg.H * cfg.I
    b, _ = bench.gemm_algorithmic_bytes(cfg, "gemm1_swiglu", cfg.E)
    assert b / (bench.PEAK_HBM_GBS * 1e9) > flops / (bench.PEAK_TFLOPS[cfg.dtype] * 1e12)
    cfg = get_config("qwen3_30b_a3b_bf16")
    flops = 4 * cfg.T * cfg.k * cfg.H * cfg.I
    b, _ = bench.gemm_algorithmic_bytes(cfg, "gemm1_swiglu", cfg.E)
    assert b / (bench.PEAK_HBM_GBS * 1e9) < flops / (bench.PEAK_TFLOPS[cfg.dtype] * 1e12)


def test_stats_markdown(tmp_path):
    csv_path = tmp_path / "kt_kernel_stats.csv"
    csv_path.write_text('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs"\n'
                        '"void moe::(anonymous namespace)::gemm_bf16_kernel<256, 128, 4, 2, true, 0, false>'
                        '(moe::(anonymous namespace)::Params)",7,3500000,500000.0,60.0,480000,520000\n')
    log = tmp_path / "run.log"
    log.write_text("noise\n" + json.dumps({"value": 1.0, "unit": "TFLOP/s", "steps": 5, "warmup": 2,
                                           "stages_us": {"gemm1_swiglu": 499.0}}) + "\n")
    out = tmp_path / "summary.md"
    bench.stats_markdown(str(csv_path), "title", "the command", str(out), str(log))
    text = out.read_text()
    assert "`gemm_bf16_kernel<256, 128, 4, 2, true, 0, false>` | 7 | 500.0 |" in text
    assert "| gemm1_swiglu | 499.0 |" in text and "the command" in text


def test_src_hash_ignores_comments(tmp_path, monkeypatch):
    csrc = tmp_path / "mixture_experts_routed_top_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "moe_common.cuh").write_text("int common;\n")
    (csrc / "k.hip").write_text("// header\nint a = 1;  // note\n/* block\n comment */\nint b = 2;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench._src_hash("k.hip")
    (csrc / "k.hip").write_text("// other header\n\nint a = 1;\nint b = 2;  /* x */\n")
    assert bench._src_hash("k.hip") == h0
    (csrc / "k.hip").write_text("int a = 1;\nint b = 3;\n")
    assert bench._src_hash("k.hip") != h0


def test_write_counters(tmp_path, monkeypatch):
    """The SQ counter record: GRBM_GUI_ACTIVE summed over 8 XCDs gives the
    clock over the dispatch time; MFMA busy over 1024 SIMDs, LDS activity
    over 256 CUs; averaged over dispatches; ignored once the source changes."""
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "_src_hash", lambda fname: "h1")
    name = "void moe::(anonymous namespace)::gemm_bf16_kernel<256, 128, 4, 2, true, 0, false>(Params)"
    cyc = 900_000                      # per XCD: 2.0 GHz over a 450 us dispatch
    vals = {"GRBM_GUI_ACTIVE": 8 * cyc, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * cyc * 1024,
            "SQ_INSTS_VALU_MFMA_MOPS_BF16": 1000.0, "SQ_INSTS_VALU_MFMA_MOPS_F8": 0.0,
            "SQ_INSTS_VALU_MFMA_MOPS_F6F4": 0.0, "SQ_LDS_IDX_ACTIVE": 0.4 * cyc * 256,
            "SQ_LDS_BANK_CONFLICT": 0.1 * cyc * 256, "SQ_BUSY_CU_CYCLES": 1.0}
    lines = ['"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"']
    for d in (1, 2):
        lines += [f'{d},"{name}","{c}",{v},1000,{1000 + 450_000}' for c, v in vals.items()]
    csv_path = tmp_path / "pmc_counter_collection.csv"
    csv_path.write_text("\n".join(lines) + "\n")
    bench.write_counters("qwen3_30b_a3b_bf16", str(csv_path), "the command")
    rec = json.load(open(tmp_path / "profiles" / "gemm1_swiglu_qwen3_30b_a3b_bf16_sq_counters.json"))
    assert rec["launches"] == 2 and rec["duration_us"] == 450.0
    assert rec["clock_ghz"] == 2.0 and rec["mfma_busy"] == 0.5
    assert rec["lds_active"] == 0.4 and rec["lds_bank_conflict_share"] == 0.25
    assert rec["mfma_flop_counted"] == 512_000 and rec["command"] == "the command"
    assert bench._counters("qwen3_30b_a3b_bf16", "gemm1_swiglu", 0)["mfma_busy"] == 0.5
    monkeypatch.setattr(bench, "_src_hash", lambda fname: "h2")
    assert bench._counters("qwen3_30b_a3b_bf16", "gemm1_swiglu", 0) is None


def test_write_counters_adds_the_kernels_of_one_call(tmp_path, monkeypatch):
    """A call that launches two kernels (the MX GEMM1's two column ranges):
    each kernel is averaged over its dispatches and the two are added."""
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "_src_hash", lambda fname: "h1")
    names = ["void moe::(anonymous namespace)::gemm_scaled_kernel<128, 256, 4, 2, true, 2, 2, 1, 1>(Params)",
             "void moe::(anonymous namespace)::gemm_scaled_kernel<128, 128, 4, 2, true, 2, 2, 1, 1>(Params)"]
    lines = ['"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"']
    d = 0
    for step in range(3):
        for name, cyc, ns in ((names[0], 800_000, 400_000), (names[1], 200_000, 100_000)):
            d += 1
            for c in bench.SQ_SET:
                v = {"GRBM_GUI_ACTIVE": 8 * cyc, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * cyc * 1024}.get(c, 0.0)
                lines.append(f'{d},"{name}","{c}",{v},0,{ns}')
    csv_path = tmp_path / "p.csv"
    csv_path.write_text("\n".join(lines) + "\n")
    bench.write_counters("mxfp4_moe_t16384", str(csv_path), "cmd")
    rec = json.load(open(tmp_path / "profiles" / "gemm1_swiglu_mxfp4_moe_t16384_sq_counters.json"))
    assert rec["kernels_per_call"] == 2 and rec["launches"] == 6
    assert rec["duration_us"] == 500.0 and rec["clock_ghz"] == 2.0 and rec["mfma_busy"] == 0.5
