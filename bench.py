"""Routed MoE-MLP forward throughput on one MI355X.

A step is one whole forward over one batch of synthetic input, with every
step of the path on the GPU: route -> align_sort -> [quantise x] ->
GEMM1 + SwiGLU -> GEMM2 -> combine. Throughput is the routed GEMM FLOPs
(6 * T * k * H * I per step) over the measured time. Inputs and prepared
weights are resident in HBM before the timed region starts.

Prints one JSON line. Default workload: the Qwen3-30B-A3B-shaped BF16 MoE at
T=8192 tokens (H=2048, 128 experts, top-8, I=768), uniform routing.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {0: 2500.0, 1: 5000.0, 2: 5000.0}      # MI355X dense MFMA: bf16, fp8, fp8 (MX f8f6f4 at fp8 rate)
PEAK_FP4_TFLOPS = 10100.0
PEAK_HBM_GBS = 8000.0
DTYPE_NAME = {0: "bf16", 1: "fp8_e4m3 (128-block scales)", 2: "mxfp4 weights x mxfp8 activations"}
# The pages' own 1-GPU forward figure for this workload (other hardware, context only):
# Liger-Kernel PR #1463, MoEBenchmark results, H200, Qwen3-30B-A3B, T=8192, BF16 forward.
PAGE_FIGURES = {"qwen3_30b_a3b_bf16": (354.38, "H200 1-GPU BF16 forward, Liger-Kernel PR #1463 MoEBenchmark"),
                 "llama4_scout_bf16": (511.36, "H200 1-GPU BF16 forward, Liger-Kernel PR #1463 MoEBenchmark")}
PAGE_FIGURES_BWD = {
    "qwen3_30b_a3b_bf16": (199.28, "H200 1-GPU BF16 backward, Liger-Kernel PR #1463 MoEBenchmark"),
    "llama4_scout_bf16": (299.54, "H200 1-GPU BF16 backward, Liger-Kernel PR #1463 MoEBenchmark")}
KERNEL_SRC = {"gemm1_swiglu": {0: "gemm_bf16.hip", 1: "gemm_scaled.hip", 2: "gemm_scaled.hip"},
              "gemm1_relu2": {0: "gemm_bf16.hip"},
              "gemm2_down": {0: "gemm_bf16.hip", 1: "gemm_scaled.hip", 2: "gemm_scaled.hip"}}
GEMM1_STAGE = {0: "gemm1_swiglu", 1: "gemm1_relu2"}     # by activation


def _src_hash(fname: str) -> str:
    """Hash of a kernel source and the common header, comments and blank lines
    left out (a comment edit does not change what the counters measured)."""
    import re
    path = os.path.join(ROOT, "mixture_experts_routed_top_amd", "csrc", fname)
    h = hashlib.sha256()
    for f in (path, os.path.join(os.path.dirname(path), "moe_common.cuh")):
        text = re.sub(r"/\*.*?\*/", "", open(f).read(), flags=re.S)
        lines = [re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines()]
        h.update("\n".join(ln for ln in lines if ln.strip()).encode())
    return h.hexdigest()[:16]


def _traffic(workload: str, kernel: str, dtype: int):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("src_hash") != _src_hash(KERNEL_SRC[kernel][dtype]):
        return None
    return rec.get("bytes_per_launch")


# ----------------------------------------------------------------- HBM traffic
# rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE give KiB per dispatch; each is scaled
# by what the same counter reads for a plain streaming copy of known size (a
# torch negation: reads N bytes, writes N bytes), run in the same process.
COPY_KERNEL_KEY = "neg"


def _kernel_role(name: str):
    """Which GEMM of the path a profiled kernel name is, or None."""
    if "gemm_bf16_kernel<" not in name and "gemm_scaled_kernel<" not in name:
        return None
    args = name.split("<", 1)[1].split(">", 1)[0]
    return "gemm1" if "true" in args else "gemm2_down"


def _read_counter(csv_path: str, counter: str):
    import csv
    per_kernel = {}
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        per_kernel.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return per_kernel


def write_traffic(workload: str, fetch_csv: str, write_csv: str, copy_mib: int, command: str):
    """Turn two counter passes of `bench.py --copy-probe-mib N` into the
    per-launch HBM byte records that the roofline object reports."""
    from workloads import get_config
    cfg = get_config(workload)
    fetch, write = _read_counter(fetch_csv, "FETCH_SIZE"), _read_counter(write_csv, "WRITE_SIZE")
    nbytes = copy_mib << 20
    copy_f = [v for k, vs in fetch.items() if COPY_KERNEL_KEY in k for v in vs]
    copy_w = [v for k, vs in write.items() if COPY_KERNEL_KEY in k for v in vs]
    if not copy_f or not copy_w:
        raise SystemExit("no copy-probe dispatch in the counter files")
    f_fac = nbytes / (1024.0 * sum(copy_f) / len(copy_f))
    w_fac = nbytes / (1024.0 * sum(copy_w) / len(copy_w))
    out = []
    for role in ("gemm1", "gemm2_down"):
        # a GEMM call may launch more than one kernel (the MX GEMM1 and the
        # BF16 squared-ReLU GEMM1 cover their last columns in a second launch):
        # average each kernel over its dispatches, then add the kernels of one call
        fks = {k: vs for k, vs in fetch.items() if _kernel_role(k) == role}
        wks = {k: vs for k, vs in write.items() if _kernel_role(k) == role}
        fk = [v for vs in fks.values() for v in vs]
        wk = [v for vs in wks.values() for v in vs]
        if role == "gemm1":
            role = GEMM1_STAGE[cfg.act]
        if not fk or not wk:
            continue
        f_kib = sum(sum(vs) / len(vs) for vs in fks.values())
        w_kib = sum(sum(vs) / len(vs) for vs in wks.values())
        rec = {"kernel": role, "workload": workload, "src_hash": _src_hash(KERNEL_SRC[role][cfg.dtype]),
               "fetch_kib_per_launch": round(f_kib, 1), "write_kib_per_launch": round(w_kib, 1),
               "copy_probe_bytes": nbytes, "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4),
               "bytes_per_launch": int(f_kib * 1024 * f_fac + w_kib * 1024 * w_fac),
               "launches": [len(fk), len(wk)], "command": command}
        path = os.path.join(ROOT, "profiles", f"{role}_{workload}_hbm_traffic.json")
        with open(path, "w") as fh:
            json.dump(rec, fh, indent=1)
        out.append(rec)
    print(json.dumps(out))


# rocprofv3 --pmc of SQ_* / GRBM_GUI_ACTIVE: GRBM_GUI_ACTIVE comes summed over
# the 8 XCDs (per-XCD busy cycles = value / 8, which over the dispatch's
# duration gives the clock the kernel ran at); the SQ counters are summed over
# every CU (LDS) or SIMD (MFMA busy).
N_XCD, N_CU, N_SIMD = 8, 256, 1024
SQ_SET = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F8",
          "SQ_INSTS_VALU_MFMA_MOPS_F6F4", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_BUSY_CU_CYCLES",
          "GRBM_GUI_ACTIVE")


def _counters(workload: str, kernel: str, dtype: int):
    """MFMA / LDS utilisation of a kernel from the committed counter record,
    or None when there is none or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_sq_counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("src_hash") != _src_hash(KERNEL_SRC[kernel][dtype]):
        return None
    return {k: rec[k] for k in ("mfma_busy", "clock_ghz", "lds_active", "lds_bank_conflict_share")}


def write_counters(workload: str, csv_path: str, command: str):
    """Turn one rocprofv3 --pmc pass of SQ_SET into per-launch MFMA / LDS
    records of the two grouped GEMMs (profiles/<kernel>_<workload>_sq_counters.json)."""
    import csv
    from workloads import get_config
    cfg = get_config(workload)
    per = {}
    for r in csv.DictReader(open(csv_path)):
        role = _kernel_role(r["Kernel_Name"])
        if role is None:
            continue
        d = per.setdefault(role, {}).setdefault(r["Kernel_Name"], {}).setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["_ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    out = []
    for role, kernels in per.items():
        name = GEMM1_STAGE[cfg.act] if role == "gemm1" else role
        # one call may launch several kernels (see write_traffic): average each
        # over its dispatches and add them, so every share below is of the
        # call's total cycles
        avg = {c: sum(sum(d[c] for d in disp.values()) / len(disp) for disp in kernels.values())
               for c in SQ_SET + ("_ns",)}
        disp = {k: d for kd in kernels.values() for k, d in kd.items()}
        cyc = avg["GRBM_GUI_ACTIVE"] / N_XCD
        mops = avg["SQ_INSTS_VALU_MFMA_MOPS_BF16"] + avg["SQ_INSTS_VALU_MFMA_MOPS_F8"] + \
            avg["SQ_INSTS_VALU_MFMA_MOPS_F6F4"]
        rec = {"kernel": name, "workload": workload, "src_hash": _src_hash(KERNEL_SRC[name][cfg.dtype]),
               "launches": len(disp), "kernels_per_call": len(kernels), "duration_us": round(avg["_ns"] / 1e3, 1),
               "clock_ghz": round(cyc / avg["_ns"], 3),
               "mfma_busy": round(avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * N_SIMD), 4),
               "mfma_flop_counted": int(mops * 512),
               "lds_active": round(avg["SQ_LDS_IDX_ACTIVE"] / (cyc * N_CU), 4),
               "lds_bank_conflict_share": round(avg["SQ_LDS_BANK_CONFLICT"] / max(avg["SQ_LDS_IDX_ACTIVE"], 1), 4),
               "counters_per_launch": {c: avg[c] for c in SQ_SET}, "command": command}
        path = os.path.join(ROOT, "profiles", f"{name}_{workload}_sq_counters.json")
        with open(path, "w") as fh:
            json.dump(rec, fh, indent=1)
        out.append(rec)
    print(json.dumps(out))


def stats_markdown(csv_path: str, title: str, command: str, out_path: str, bench_log: str = ""):
    """A short markdown table of a rocprofv3 --stats kernel summary, with the
    bench line the same profiled run printed (its HIP-event stage times)."""
    import csv

    def short(n):
        n = n.replace("moe::(anonymous namespace)::", "").replace("void ", "")
        depth, out = 0, ""
        for ch in n:
            if ch == "(" and depth == 0:
                break
            depth += (ch == "<") - (ch == ">")
            out += ch
        return out.strip()

    lines = [f"# {title}", "", "Command (run from /tmp on one MI355X, repository at $R):", "", "```", command, "```", "",
             "Times in microseconds over every dispatch of the run (warm-up steps included).", "",
             "| kernel | calls | average us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in csv.DictReader(open(csv_path)):
        lines.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    if bench_log:
        recs = [json.loads(l) for l in open(bench_log) if l.startswith("{")]
        if recs:
            r = recs[-1]
            lines += ["", f"The same run's bench line: {r['value']} {r['unit']}, {r['steps']} timed steps after "
                      f"{r['warmup']} warm-up steps; average time of each stage over the timed steps, from HIP "
                      "events on the launch stream (us):", "",
                      "| stage | us |", "|---|---|"]
            lines += [f"| {k} | {v} |" for k, v in r["stages_us"].items()]
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def copy_probe(mib: int):
    import torch
    src = torch.ones((mib << 20) // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def cpu_baseline(cfg, inp, budget_s: float = 15.0, backward: bool = False):
    """The oracle as it stands, timed on this host on a bounded prefix of the
    same batch (same weights, the first T' tokens), scaled to TFLOP/s
    (backward=True: the oracle's backward, which also recomputes the forward
    it needs, counted at the backward's FLOPs only)."""
    import numpy as np
    from oracle import moe as O
    from workloads import to_f64

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    w1 = to_f64(inp.w1)
    w2 = to_f64(inp.w2)
    dout = None
    if backward:
        from workloads import make_dout
        dout = to_f64(make_dout(cfg, 0))

    def run(t):
        logits = inp.logits[:t].numpy()
        x = to_f64(inp.x[:t])
        t0 = time.perf_counter()
        if backward:
            O.moe_backward(logits, x, w1, w2, dout[:t], cfg.k, cfg.score, block_m=16, n_shared=cfg.n_shared)
        else:
            O.moe_forward(logits, x, w1, w2, cfg.k, cfg.score, cfg.dtype, block_m=16, act=cfg.act,
                          n_shared=cfg.n_shared)
        return time.perf_counter() - t0

    # grow the token prefix until one oracle run takes about budget_s
    t_sample = min(cfg.T, 64)
    dt = run(t_sample)
    while dt < 0.5 * budget_s and t_sample < cfg.T:
        t_sample = int(min(cfg.T, max(t_sample + 1, t_sample * budget_s / max(dt, 1e-3))))
        dt = run(t_sample)
    flops = (2 if backward else 1) * cfg.flops // cfg.T * t_sample
    what = "backward" if backward else "forward"
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 numpy oracle {what} on the first {t_sample} of {cfg.T} tokens of the same batch "
                      f"(same weights), {dt:.2f} s"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen3_30b_a3b_bf16")
    ap.add_argument("--tokens", type=int, default=None, help="override T (parity-size runs)")
    ap.add_argument("--block-m", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run a plain streaming copy of this many MiB (HBM counter calibration)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM traffic records from two rocprofv3 counter passes and exit")
    ap.add_argument("--write-counters", metavar="SQ_CSV",
                    help="write the MFMA / LDS counter records from a rocprofv3 pass of the SQ counters and exit")
    ap.add_argument("--traffic-command", default="", help="the command that made the profile")
    ap.add_argument("--sweep", choices=("grid", "tokens"), default=None,
                    help="throughput sweep, one JSON line per shape: the BF16 parameter grid or the token sweep")
    ap.add_argument("--fused-combine", action="store_true",
                    help="BF16: run GEMM2 with the weighted combine fused into its epilogue")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward of the BF16 SwiGLU layer instead of the forward")
    ap.add_argument("--stats-md", nargs=3, metavar=("STATS_CSV", "TITLE", "OUT_MD"),
                    help="write a markdown summary of a rocprofv3 --stats kernel table and exit")
    ap.add_argument("--bench-log", default="", help="with --stats-md: the profiled run's output (its bench line)")
    a = ap.parse_args(argv)

    if a.stats_md:
        stats_markdown(a.stats_md[0], a.stats_md[1], a.traffic_command, a.stats_md[2], a.bench_log)
        return 0
    if a.write_counters:
        write_counters(a.workload, a.write_counters, a.traffic_command)
        return 0
    if a.write_traffic:
        write_traffic(a.workload, a.write_traffic[0], a.write_traffic[1], a.copy_probe_mib or 1024,
                      a.traffic_command)
        return 0

    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the routed forward here is the "
              "single-GPU path and has no multi-GPU mode.", file=sys.stderr)
        return 2

    import torch

    torch.cuda.set_device(0)
    if a.copy_probe_mib:
        copy_probe(a.copy_probe_mib)
    if a.sweep:
        return sweep(a)

    from workloads import get_config, make_inputs
    cfg = get_config(a.workload)
    if a.tokens:
        cfg = cfg.with_(T=a.tokens)
    inp = make_inputs(cfg)
    if a.backward:
        rec = measure_backward(cfg, inp, a.steps, a.warmup)
        base = PAGE_FIGURES_BWD.get(cfg.name) if not a.tokens else None
    else:
        rec = measure(cfg, inp, a.steps, a.warmup, a.block_m, fused_combine=a.fused_combine)
        base = PAGE_FIGURES.get(cfg.name) if not a.tokens else None
    rec["vs_baseline"] = round(rec["value"] / base[0], 4) if base else None
    rec["baseline_ref"] = f"{base[0]} TFLOP/s, {base[1]} (other hardware, context only)" if base else None
    if not a.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, inp, backward=a.backward)
    print(json.dumps(rec), flush=True)
    return 0


def _time_stages(stage_fns, steps: int, warmup: int):
    """Run `warmup` untimed passes, then time `steps` passes of the stage
    functions, with events on the launch stream around every stage."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        for _, f in stage_fns:
            f()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stage_fns) + 1)] for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for s in range(steps):
        ev[s][0].record(stream)
        for i, (_, f) in enumerate(stage_fns):
            f()
            ev[s][i + 1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / steps
    stage_us = {}
    for i, (name, _) in enumerate(stage_fns):
        stage_us[name] = round(1000.0 * sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)) / steps, 2)
    steps_ms = sorted(ev[s][0].elapsed_time(ev[s][-1]) for s in range(steps))
    step_stats = {"median": round(steps_ms[len(steps_ms) // 2], 4), "min": round(steps_ms[0], 4),
                  "p90": round(steps_ms[min(len(steps_ms) - 1, int(0.9 * len(steps_ms)))], 4)}
    return ms, stage_us, step_stats, wall


def _config(cfg, plan):
    return {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "k": cfg.k, "I": cfg.I,
            "n_shared": cfg.n_shared, "activation": "swiglu" if cfg.act == 0 else "relu2",
            "routing": cfg.routing, "score": "softmax" if cfg.score == 0 else "sigmoid",
            "numeric_path": DTYPE_NAME[cfg.dtype], "block_m": plan.block_m, "parallelism": "none (1 GPU)",
            "fused_combine": plan.counters is not None}


def measure(cfg, inp, steps: int, warmup: int, block_m=None, data=None, fused_combine=False) -> dict:
    """Time `steps` whole forwards of workload cfg on inputs inp (after
    `warmup` untimed ones) and build the result record."""
    import torch
    import mixture_experts_routed_top_amd as M

    dev = "cuda:0"
    layer = M.MoeLayer(cfg.dtype, inp.w1.to(dev), inp.w2.to(dev), cfg.k, cfg.score, cfg.act, cfg.n_shared,
                       fused_combine=fused_combine)
    x, logits = inp.x.to(dev), inp.logits.to(dev)
    plan = layer.plan(cfg.T, block_m=block_m)
    torch.cuda.synchronize()

    # timed region: K whole forwards
    ms, stage_us, step_stats, wall = _time_stages(_stage_fns(layer, plan, x, logits), steps, warmup)
    flops = cfg.flops
    value = flops / (ms / 1e3) / 1e12
    # the compute-only rate (x already quantised: every stage but quantize_x)
    # next to the end-to-end one
    compute_us = sum(v for n, v in stage_us.items() if n != "quantize_x")

    # roofline of the dominant kernel (largest average duration)
    g1 = GEMM1_STAGE[cfg.act]
    g2 = "gemm2_down_combine" if "gemm2_down_combine" in stage_us else "gemm2_down"
    dom = max((g1, g2), key=lambda n: stage_us[n])
    fl_mult = {"gemm1_swiglu": 4, "gemm1_relu2": 2, "gemm2_down": 2, "gemm2_down_combine": 2}[dom]
    dom_flops = fl_mult * cfg.T * (cfg.k + cfg.n_shared) * cfg.H * cfg.I   # rows the kernel computes
    peak = PEAK_TFLOPS[cfg.dtype]
    e_used = int((plan.sort.counts > 0).sum().item())
    dom_bytes, bytes_note = gemm_algorithmic_bytes(cfg, dom, e_used)
    # the binding resource: MFMA time of the FLOPs at peak, or HBM time of the
    # bytes the kernel must move at least once (small token counts stream the
    # weights of every expert used and do little arithmetic on them)
    if dom_bytes / (PEAK_HBM_GBS * 1e9) > dom_flops / (peak * 1e12):
        achieved = dom_bytes / (stage_us[dom] * 1e-6) / 1e9
        roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = dom_flops / (stage_us[dom] * 1e-6) / 1e12
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
    roofline.update({"traffic": _traffic(cfg.name, dom, cfg.dtype), "counters": _counters(cfg.name, dom, cfg.dtype),
                     "avg_launch_us": stage_us[dom],
                     "algorithmic": f"{fl_mult}*T*(k+shared)*H*I = {dom_flops} FLOP per launch; "
                                    f"{bytes_note} = {dom_bytes} B per launch"})

    rec = {
        "metric": "routed MoE-MLP forward TFLOP/s on 1 MI355X (+% of dtype MFMA peak)",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == 0 else ("fp8" if cfg.dtype == 1 else "mxfp4xmxfp8"),
        "data": data or "synthetic (seeded N(0,1) tokens, N(0,sigma) bf16 weights, router logits x.Wr)",
        "config": _config(cfg, plan),
        "pct_of_dtype_peak": round(100 * value / peak, 2),
        "step_ms": step_stats,
        "compute_tflops": round(flops / (compute_us * 1e-6) / 1e12, 2),
        "stages_us": stage_us,
        "wall_s_timed": round(wall, 4),
        "roofline": roofline,
    }
    if cfg.dtype == 2:
        rec["pct_of_fp4_peak"] = round(100 * value / PEAK_FP4_TFLOPS, 2)
    return rec


def gemm_algorithmic_bytes(cfg, kernel: str, e_used: int):
    """Bytes a grouped GEMM of the forward must move at least once per launch:
    the weights (and block scales) of the e_used experts that received rows,
    the token operand read once, and its output written once (GEMM1: the
    intermediate h of the A = T*(k+shared) real rows; GEMM2: h read, Y
    written in bf16). Pad rows are not counted."""
    A, H, I = cfg.T * (cfg.k + cfg.n_shared), cfg.H, cfg.I
    if cfg.dtype == 0:                      # bf16 everywhere
        val, scale_w, scale_a = 2.0, 0.0, 0.0
    elif cfg.dtype == 1:                    # E4M3, fp32 per 128x128 (weights) / 1x128 (tokens)
        val, scale_w, scale_a = 1.0, 4.0 / (128 * 128), 4.0 / 128
    else:                                   # E2M1 weights / E4M3 tokens, one E8M0 byte per 32
        val, scale_w, scale_a = 1.0, 1.0 / 32, 1.0 / 32
    wval = 0.5 if cfg.dtype == 2 else val   # weight element bytes
    if kernel.startswith("gemm1"):
        rows = cfg.w1_rows
        w = e_used * rows * H * (wval + scale_w)
        x = cfg.T * H * (val + scale_a)
        h = A * I * (val + scale_a)
        return int(w + x + h), f"{e_used} experts x W1 ({rows}x{H}) + x (T x H) + h (A x I)"
    w = e_used * H * I * (wval + scale_w)
    h = A * I * (val + scale_a)
    y = A * H * 2
    return int(w + h + y), f"{e_used} experts x W2 ({H}x{I}) + h (A x I) + Y (A x H, bf16)"


def bwd_algorithmic_bytes(cfg, kernel: str, e_used: int):
    """Bytes a backward GEMM must move at least once per launch (bf16 rows of
    the A = T*(k+shared) real assignments, weights of the experts that
    received rows, fp32 weight gradients of every expert)."""
    A, H, I, E = cfg.T * (cfg.k + cfg.n_shared), cfg.H, cfg.I, cfg.E_total
    if kernel == "gemm_dh":
        return A * H * 2 + e_used * H * I * 2 + 2 * A * 2 * I * 2, "dY + W2 (experts used) + gu + dGU"
    if kernel == "gemm_dx":
        return A * 2 * I * 2 + e_used * 2 * I * H * 2 + A * H * 2, "dGU + W1 (experts used) + dx rows"
    if kernel == "wgrad_w2":
        return A * I * 2 + A * H * 2 + E * H * I * 4, "h + dY + dW2 (fp32)"
    return A * H * 2 + A * 2 * I * 2 + E * 2 * I * H * 4, "x rows + dGU + dW1 (fp32)"


# FLOPs per launch of each backward GEMM, in units of T*(k+shared)*H*I
BWD_GEMM_FLOPS = {"gemm_dh": 2, "gemm_dx": 4, "wgrad_w2": 2, "wgrad_w1": 4}


def measure_backward(cfg, inp, steps: int, warmup: int, data=None) -> dict:
    """Time `steps` backward passes of the BF16 SwiGLU layer (after one
    training forward that saves what they read): combine backward, router
    backward, dGU, dx rows, dx, row gather, dW2, dW1. Throughput counts the
    routed backward GEMM FLOPs, 12 * T * k * H * I per step (twice the
    forward's)."""
    import torch
    import mixture_experts_routed_top_amd as M
    from workloads import make_dout

    if cfg.dtype != 0 or cfg.act != 0:
        raise SystemExit("the backward is implemented for the BF16 SwiGLU layer")
    dev = "cuda:0"
    layer = M.MoeLayer(cfg.dtype, inp.w1.to(dev), inp.w2.to(dev), cfg.k, cfg.score, cfg.act, cfg.n_shared)
    x, logits = inp.x.to(dev), inp.logits.to(dev)
    dout = make_dout(cfg, 0).to(dev)
    p = layer.plan(cfg.T, train=True)
    layer.forward_train(x, logits, p)
    torch.cuda.synchronize()
    tb, H, I = p.train, layer.H, layer.I
    fns = [("backward_combine", lambda: M.moe_backward_combine(dout, p.w, p.y, p.sort, tb.dy, tb.dw)),
           ("route_backward", lambda: M.moe_route_backward(p.w, p.ids, tb.dw, layer.E - layer.n_shared,
                                                           layer.k_routed, layer.score, layer.n_shared,
                                                           tb.dlogits)),
           ("gemm_dh", lambda: M.moe_grouped_gemm_dh(tb.dy, layer.w2, tb.gu, p.sort, H, I, tb.dgu)),
           ("gemm_dx", lambda: M.moe_grouped_gemm_dx(tb.dgu, layer.w1, p.sort, H, I, tb.dx_rows)),
           ("dx_reduce", lambda: M.moe_combine(tb.dx_rows, tb.ones, tb.dx)),
           ("gather_rows", lambda: M.moe_gather_rows(x, p.sort, tb.x_sorted)),
           ("wgrad_w2", lambda: M.moe_grouped_gemm_wgrad(p.h, tb.dy, p.sort, tb.dw2)),
           ("wgrad_w1", lambda: M.moe_grouped_gemm_wgrad(tb.x_sorted, tb.dgu, p.sort, tb.dw1))]
    ms, stage_us, step_stats, wall = _time_stages(fns, steps, warmup)
    unit = cfg.T * (cfg.k + cfg.n_shared) * cfg.H * cfg.I
    flops = 2 * cfg.flops
    value = flops / (ms / 1e3) / 1e12
    dom = max(BWD_GEMM_FLOPS, key=lambda n: stage_us[n])
    dom_flops = BWD_GEMM_FLOPS[dom] * unit
    peak = PEAK_TFLOPS[0]
    e_used = int((p.sort.counts > 0).sum().item())
    dom_bytes, bytes_note = bwd_algorithmic_bytes(cfg, dom, e_used)
    if dom_bytes / (PEAK_HBM_GBS * 1e9) > dom_flops / (peak * 1e12):
        achieved = dom_bytes / (stage_us[dom] * 1e-6) / 1e9
        rl = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
              "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = dom_flops / (stage_us[dom] * 1e-6) / 1e12
        rl = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
              "frac": round(achieved / peak, 4)}
    gemm_tflops = {n: round(BWD_GEMM_FLOPS[n] * unit / (stage_us[n] * 1e-6) / 1e12, 2) for n in BWD_GEMM_FLOPS}
    return {
        "metric": "routed MoE-MLP backward TFLOP/s on 1 MI355X (+% of dtype MFMA peak)",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": data or "synthetic (seeded N(0,1) tokens and output gradient, N(0,sigma) bf16 weights, "
                        "router logits x.Wr)",
        "config": _config(cfg, p),
        "pct_of_dtype_peak": round(100 * value / peak, 2),
        "step_ms": step_stats, "stages_us": stage_us, "gemm_tflops": gemm_tflops, "wall_s_timed": round(wall, 4),
        "roofline": {"kernel": dom, **rl, "traffic": None, "avg_launch_us": stage_us[dom],
                     "algorithmic": f"{BWD_GEMM_FLOPS[dom]}*T*(k+shared)*H*I = {dom_flops} FLOP per launch; "
                                    f"{bytes_note} = {dom_bytes} B per launch"},
    }


def sweep(a) -> int:
    """One JSON line per shape: the BF16 parameter grid (T=8192, D=I in
    {2048, 4096}, E in {8..128}, top-K in {1, 2, 4, 8}) or the token sweep of
    the named BF16 shapes (T = 1024 .. 16384). Inputs drawn on the GPU."""
    import torch
    from workloads import P5_GRID, get_config, make_inputs_device

    if a.sweep == "grid":
        cfgs = [get_config(n) for n in P5_GRID]
    elif a.sweep == "tokens":
        cfgs = [get_config(n).with_(T=t) for n in ("qwen3_30b_a3b_bf16", "llama4_scout_bf16")
                for t in (1024, 2048, 4096, 8192, 16384)]
    else:
        raise SystemExit(f"unknown sweep {a.sweep!r}")
    for cfg in cfgs:
        inp = make_inputs_device(cfg, "cuda:0")
        rec = measure(cfg, inp, a.steps, a.warmup,
                      data="synthetic, drawn on the GPU (seeded torch generator; same distributions)")
        print(json.dumps({"sweep": a.sweep, "workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "k": cfg.k,
                          "I": cfg.I, "value": rec["value"], "unit": "TFLOP/s", "ms_per_step": rec["ms_per_step"],
                          "pct_of_dtype_peak": rec["pct_of_dtype_peak"], "block_m": rec["config"]["block_m"],
                          "stages_us": rec["stages_us"]}), flush=True)
        del inp, rec
        torch.cuda.empty_cache()
    return 0


def _stage_fns(layer, plan, x, logits):
    import mixture_experts_routed_top_amd as M
    d = layer.dtype
    route = (lambda: M.moe_route_shared(logits, layer.k_routed, layer.score, layer.n_shared, plan.ids, plan.w)) \
        if layer.n_shared else (lambda: M.moe_route(logits, layer.k, layer.score, plan.ids, plan.w))
    fns = [("route", route),
           ("align_sort", lambda: M.moe_align_sort(plan.ids, layer.E, plan.block_m, out=plan.sort))]
    if d == M.DTYPE_FP8_BLOCK128:
        fns.append(("quantize_x", lambda: M.moe_quantize_fp8(x, 1, plan.xq, plan.xs)))
        a, a_s = plan.xq, plan.xs
    elif d == M.DTYPE_MXFP4W_MXFP8A:
        fns.append(("quantize_x", lambda: M.moe_quantize_mxfp8(x, plan.xq, plan.xs)))
        a, a_s = plan.xq, plan.xs
    else:
        a, a_s = x, None
    gemm1 = M.moe_grouped_gemm_swiglu if layer.act == M.ACT_SWIGLU else M.moe_grouped_gemm_relu2
    fns.append((GEMM1_STAGE[layer.act], lambda: gemm1(d, a, a_s, layer.w1, layer.w1_scale, plan.sort,
                                                      layer.H, layer.I, plan.h, plan.h_scale, ws=plan.ws)))
    if layer.fused_combine:
        fns.append(("gemm2_down_combine", lambda: M.moe_grouped_gemm_down_combine(
            d, plan.h, plan.h_scale, layer.w2, layer.w2_scale, plan.sort, layer.H, layer.I, plan.w, plan.counters,
            plan.y, plan.out)))
        return fns
    fns.append(("gemm2_down", lambda: M.moe_grouped_gemm_down(d, plan.h, plan.h_scale, layer.w2, layer.w2_scale,
                                                                plan.sort, layer.H, layer.I, plan.y, ws=plan.ws)))
    fns.append(("combine", lambda: M.moe_combine(plan.y, plan.w, plan.out)))
    return fns


if __name__ == "__main__":
    sys.exit(main())
