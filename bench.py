#!/usr/bin/env python3
"""Benchmark of the MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixtral]

A step is one moe_forward (route, dispatch, grouped gate/up GEMM with the
SwiGLU epilogue, grouped down GEMM, combine) over one batch of T tokens of
seeded synthetic input already resident in HBM. Prints ONE JSON line on
stdout; a per-stage table goes to stderr.

Workload (default): the Mixtral-shape layer, T=4096 tokens, D=4096, E=8
experts, top-2, SwiGLU F=14336, bf16 activations and weights with fp32
accumulation, softmax -> top-k -> renormalised, per-expert logit offsets
~N(0, 0.5).
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s (1 GPU) + grouped-GEMM TFLOP/s as % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_MXFP4_TFLOPS = 10100.0  # MI355X dense fp4 MFMA
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFLOPS = 157.3     # MI355X fp32 (vector and MFMA)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_{workload}.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device copy (for counter scaling)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write profiles/kernel_trace_<workload>.txt from a rocprofv3 --stats run")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/hbm_traffic_<workload>.{json,txt} from two --pmc runs")
    ap.add_argument("--summarize-mfma", metavar="DIR",
                    help="write profiles/mfma_util_<workload>.txt from a rocprofv3 --pmc MfmaUtil run")
    ap.add_argument("--profile-command", default="",
                    help="the command that produced the profile, recorded in the summary")
    ap.add_argument("--study", choices=["dense-vs-moe", "topk"],
                    help="instead of the layer benchmark: the dense layer against an MoE of "
                         "single-linear experts, or the top-k 1/2/4 sweep (one JSON line per "
                         "measurement)")
    return ap.parse_args()


def algorithmic(cfg, A):
    """Algorithmic work of one forward (what the method must compute/move).
    With bf16 activations dispatch copies no rows (the gate/up GEMM gathers
    them from x), so its bytes are the indices alone: topk_idx read,
    slot_pos and perm_token written."""
    sx = 2 if cfg.act == 1 else 4
    T, D, E, k, F = cfg.T, cfg.D, cfg.E, cfg.k, cfg.F
    rows = 0 if cfg.act == 1 else T * D * sx + A * D * sx
    return dict(
        gate_up_flop=4.0 * D * F * A,
        down_flop=2.0 * D * F * A,
        shared_flop=6.0 * D * cfg.shared_F * T,
        route_bytes=T * D * sx + D * E * 4 + T * k * 8,
        dispatch_bytes=T * k * 8 + A * 4 + rows,
        combine_bytes=A * D * 4 + T * k * 8 + T * D * sx + (T * D * 4 if cfg.shared_F else 0),
    )


CSRC = os.path.join(ROOT, "mixture_experts_layer_25_amd", "csrc")


def roofline_kernel(cfg):
    """The gate/up kernel the workload's weight type selects, its source
    file and what bounds it."""
    if cfg.wdt == 0:  # fp32 MFMA: the same 157.3 TFLOP/s as the fp32 vector ALUs
        return {"name": "ffn_f32_gemm_kernel<true>", "src": "ffn_f32.hip", "bound": "mfma",
                "peak": PEAK_FP32_TFLOPS}
    if cfg.wdt == 3:  # e4m3 x e2m1 products run at the fp8 MFMA rate
        return {"name": "gemm_a8_kernel<0>", "src": "gemm_a8.hip", "bound": "mfma",
                "peak": PEAK_FP8_TFLOPS}
    if cfg.wdt == 2:
        return {"name": "gemm16_mx_kernel<0>", "src": "gemm16.hip", "bound": "mfma"}
    return {"name": "gemm16_kernel<0>", "src": "gemm16.hip", "bound": "mfma"}


def _sources_of(name, seen=None):
    """The kernel source and the local headers it includes, recursively."""
    seen = [] if seen is None else seen
    if name in seen or not os.path.exists(os.path.join(CSRC, name)):
        return seen
    seen.append(name)
    for inc in re.findall(r'^#include "([^"/]+)"', open(os.path.join(CSRC, name)).read(), re.M):
        _sources_of(inc, seen)
    return seen


def src_sha256(name):
    """sha256 of the code that builds the kernel: its source and the local
    headers it includes, with // comments and blank lines removed (a change
    of comments does not change the kernel; a change of code anywhere in
    those files does)."""
    h = hashlib.sha256()
    for f in sorted(_sources_of(name)):
        h.update(f.encode())
        for line in open(os.path.join(CSRC, f)).read().splitlines():
            code = line.split("//", 1)[0].rstrip()
            if code.strip():
                h.update(code.encode() + b"\n")
    return h.hexdigest()


def short_name(n):
    n = n.replace("moe::(anonymous namespace)::", "").replace("void ", "")
    if "(" in n and not n.startswith("__"):
        n = n[:n.index("(")]
    return n[:90]


def read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def find_one(d, suffix):
    hits = [os.path.join(r, f) for r, _, fs in os.walk(d) for f in fs if f.endswith(suffix)]
    if len(hits) != 1:
        raise SystemExit(f"expected one *{suffix} under {d}, found {len(hits)}")
    return hits[0]


def _arg_of(command, flag, default):
    m = re.search(re.escape(flag) + r"[ =](\d+)", command)
    return int(m.group(1)) if m else default


def summarize_trace(run_dir, workload, command):
    """rocprofv3 --kernel-trace --stats output -> profiles/kernel_trace_<workload>.txt:
    every kernel's statistics over all its dispatches, and for the roofline
    kernel the mean over the dispatches of the two timed passes of the
    benchmark (in launch order: W warm-up and K timed moe_forward steps, then
    max(1, W/2) warm-up and K timed stage-by-stage steps), the second of which
    is the live figure the benchmark reports."""
    from mixture_experts_layer_25_amd import synthetic as syn
    rows = read_csv(find_one(run_dir, "kernel_stats.csv"))
    out = os.path.join(ROOT, "profiles", f"kernel_trace_{workload}.txt")
    lines = [f"# rocprofv3 kernel-trace summary, workload {workload}",
             f"# command: {command}",
             "# durations in microseconds per dispatch",
             f"{'kernel':90s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}"]
    for r in rows:
        lines.append(f"{short_name(r['Name']):90s} {int(r['Calls']):6d} "
                     f"{float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
                     f"{float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):6.2f}")
    rk = roofline_kernel(syn.CONFIGS[workload])["name"]
    K = _arg_of(command, "--steps", 50)
    W = _arg_of(command, "--warmup", 10)
    disp = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
                  for r in read_csv(find_one(run_dir, "kernel_trace.csv"))
                  if short_name(r["Kernel_Name"]) == rk)
    dur = [(e - s) / 1e3 for s, e in disp]
    w2 = max(1, W // 2)
    fused = dur[W:W + K]
    stage = dur[W + K + w2:W + K + w2 + K]
    if len(dur) >= W + K + w2 + K:
        lines.append(f"# {rk}: {len(dur)} dispatches; mean of the {K} timed moe_forward steps "
                     f"{sum(fused) / K:.2f} us, of the {K} timed stage-by-stage steps (the "
                     f"benchmark's live roofline figure) {sum(stage) / K:.2f} us")
    open(out, "w").write("\n".join(lines) + "\n")
    print(out)


# MFMA flops per busy pipe cycle and SIMD: v_mfma_f32_16x16x32_bf16 (16384
# flops in 16 cycles), the block-scaled fp8 x fp4 MFMA (twice the rate) and
# v_mfma_f32_16x16x4_f32 (2048 flops in 32 cycles)
MFMA_FLOP_PER_CYCLE = {"gemm16": 1024, "gemm_a8": 2048, "ffn_f32_gemm": 64}
XCDS = 8


def summarize_mfma(run_dir, workload, command):
    """rocprofv3 --pmc MfmaUtil GRBM_GUI_ACTIVE -> profiles/mfma_util_<workload>.txt:
    per kernel the mean over its dispatches of MfmaUtil
    (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs), per cent), of the
    clock under load (GRBM_GUI_ACTIVE cycles, which the counter reports
    summed over the 8 XCDs, over the dispatch's duration; meaningless for
    dispatches of a few microseconds)
    and of the rate they imply for an MFMA kernel, MfmaUtil x SIMDs x flops
    per busy cycle x clock (1024 SIMDs on MI355X)."""
    from collections import defaultdict
    util, clk, dur = defaultdict(list), defaultdict(list), defaultdict(list)
    for r in read_csv(find_one(run_dir, "counter_collection.csv")):
        k = short_name(r["Kernel_Name"])
        ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        if r["Counter_Name"] == "MfmaUtil":
            util[k].append(float(r["Counter_Value"]))
            dur[k].append(ns / 1e3)
        elif r["Counter_Name"] == "GRBM_GUI_ACTIVE" and ns > 0:
            # the counter comes summed over the XCDs (8 on MI355X)
            clk[k].append(float(r["Counter_Value"]) / XCDS / ns)
    out = os.path.join(ROOT, "profiles", f"mfma_util_{workload}.txt")
    lines = [f"# MFMA pipe utilisation (MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x "
             f"SIMDs), per cent), clock under load (GRBM_GUI_ACTIVE / dispatch duration) and the "
             f"MFMA rate they imply (MfmaUtil x 1024 SIMDs x flop per busy cycle x clock), "
             f"workload {workload}",
             f"# command: {command}",
             f"{'kernel':90s} {'dispatches':>10s} {'MfmaUtil_%':>10s} {'clock_GHz':>9s} "
             f"{'avg_us':>9s} {'implied_TF':>10s}"]
    for k in sorted(util, key=lambda k: -sum(util[k]) / len(util[k])):
        u = sum(util[k]) / len(util[k])
        c = sum(clk[k]) / len(clk[k]) if clk.get(k) else float("nan")
        fpc = next((v for n, v in MFMA_FLOP_PER_CYCLE.items() if k.startswith(n)), 0)
        tf = u / 100 * 1024 * fpc * c * 1e9 / 1e12 if fpc else float("nan")
        lines.append(f"{k:90s} {len(util[k]):10d} {u:10.1f} {c:9.3f} "
                     f"{sum(dur[k]) / len(dur[k]):9.1f} {tf:10.1f}")
    open(out, "w").write("\n".join(lines) + "\n")
    print(out)


def summarize_pmc(fetch_dir, write_dir, workload, command):
    """Two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of
    `bench.py --copy-calibration` -> HBM bytes per dispatch of each kernel.
    Each counter is scaled by what it reads for the plain 256 MiB device copy
    in the same run (the largest __amd_rocclr_copyBuffer dispatch), so
    bytes = KiB x 1024 x (256 MiB / copy reading)."""
    from collections import defaultdict
    cfg_name = workload
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in read_csv(find_one(d, "counter_collection.csv"))
                if r["Counter_Name"] == counter]
        copy = max((float(r["Counter_Value"]) for r in rows
                    if r["Kernel_Name"] == "__amd_rocclr_copyBuffer"), default=0.0)
        if copy <= 0:
            raise SystemExit(f"{counter}: no calibration copy in {d}")
        scale = 256 * 1024 / copy
        per = defaultdict(list)
        for r in rows:
            per[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
        res[counter] = {"copy_kib": copy, "scale": scale,
                        "kib_per_dispatch": {k: sum(v) / len(v) for k, v in per.items()}}
    from mixture_experts_layer_25_amd import synthetic as syn
    rk = roofline_kernel(syn.CONFIGS[cfg_name])
    f = res["FETCH_SIZE"]
    w = res["WRITE_SIZE"]

    def nbytes(k):
        return (f["kib_per_dispatch"].get(k, 0.0) * f["scale"]
                + w["kib_per_dispatch"].get(k, 0.0) * w["scale"]) * 1024

    rec = {"workload": cfg_name, "kernel": rk["name"], "kernel_src": rk["src"],
           "kernel_src_sha256": src_sha256(rk["src"]),
           "fetch_scale": f["scale"], "write_scale": w["scale"],
           "bytes_per_launch": nbytes(rk["name"]), "command": command,
           "per_kernel_bytes": {k: nbytes(k) for k in sorted(set(f["kib_per_dispatch"]) |
                                                              set(w["kib_per_dispatch"]))}}
    base = os.path.join(ROOT, "profiles", f"hbm_traffic_{cfg_name}")
    json.dump(rec, open(base + ".json", "w"), indent=1)
    lines = [f"# HBM traffic per dispatch from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE, workload {cfg_name}",
             f"# command: {command}",
             f"# scaling: FETCH_SIZE x {f['scale']:.4f} (copy of 256 MiB read {f['copy_kib']:.1f} KiB), "
             f"WRITE_SIZE x {w['scale']:.4f} (copy wrote {w['copy_kib']:.1f} KiB)",
             f"# code sha256 of {rk['src']} and its headers (comments stripped): "
             f"{rec['kernel_src_sha256']}",
             f"{'kernel':90s} {'fetch_KiB':>12s} {'write_KiB':>12s} {'scaled_MB':>10s}"]
    for k, b in rec["per_kernel_bytes"].items():
        lines.append(f"{k:90s} {f['kib_per_dispatch'].get(k, 0.0):12.1f} "
                     f"{w['kib_per_dispatch'].get(k, 0.0):12.1f} {b / 1e6:10.2f}")
    open(base + ".txt", "w").write("\n".join(lines) + "\n")
    print(base + ".json")


def pct(vals, q):
    v = sorted(vals)
    i = min(len(v) - 1, max(0, int(round(q / 100.0 * (len(v) - 1)))))
    return v[i]


def _time_steps(fns, steps, warmup, stream):
    """Per-step times (ms) of running fns in order, with an event between
    the stages; returns (per_step_ms, per_stage_mean_ms)."""
    import torch
    for _ in range(warmup):
        for fn in fns:
            fn()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for evs in ev:
        evs[0].record(stream)
        for i, fn in enumerate(fns):
            fn()
            evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = [evs[0].elapsed_time(evs[-1]) for evs in ev]
    per_stage = [sum(evs[i].elapsed_time(evs[i + 1]) for evs in ev) / steps for i in range(len(fns))]
    return per_step, per_stage


def study_dense_vs_moe(args):
    """The pages' dense-versus-MoE comparison (S = 4096, D = 4096, 8 experts,
    top-2; dense 4096 x 4096, experts 4096 x 512) on this GPU."""
    import numpy as np
    import torch

    from mixture_experts_layer_25_amd import moe, studies, synthetic as syn

    T, D, E, k, n_out = 4096, 4096, 8, 2, 512
    x_h, W_r_h, W_lin_h, W_dense_h = syn.make_linear_layer_inputs(T, D, E, n_out)
    dev = "cuda"
    x = torch.from_numpy(x_h.view(np.int16)).to(dev).view(torch.bfloat16)
    W_r = torch.from_numpy(W_r_h).to(dev)
    W_lin = torch.from_numpy(W_lin_h.view(np.int16)).to(dev).view(torch.bfloat16)
    W_dense = torch.from_numpy(W_dense_h.view(np.int16)).to(dev).view(torch.bfloat16)
    cfg = moe.make_cfg(T=T, D=D, E=E, F=n_out, top_k=k, gating="softmax", renorm=True)
    lin = studies.LinearMoE(cfg, x, W_r, None, W_lin)
    dense = studies.DenseLinear(x, W_dense)
    stream = torch.cuda.current_stream()
    names = [n for n, _ in lin.stages()]
    moe_steps, moe_stages = _time_steps([f for _, f in lin.stages()], args.steps, args.warmup, stream)
    dense_steps, _ = _time_steps([dense], args.steps, args.warmup, stream)
    moe_ms = float(np.mean(moe_steps))
    dense_ms = float(np.mean(dense_steps))
    rec = {"study": "dense_vs_moe", "tokens": T, "D": D, "experts": E, "top_k": k,
           "expert_shape": [D, n_out], "dense_shape": [D, D], "dtype": "bf16",
           "dense_ms": round(dense_ms, 4), "moe_ms": round(moe_ms, 4),
           "dense_over_moe": round(dense_ms / moe_ms, 3),
           "moe_stage_ms": {n: round(v, 4) for n, v in zip(names, moe_stages)},
           "dense_tflops": round(2.0 * T * D * D / (dense_ms * 1e-3) / 1e12, 1),
           "activated_params": {"dense": D * D, "moe": k * D * n_out},
           "pages_ascend910": {"dense": 2.8, "moe": 1.5, "units": "unstated"},
           "steps": args.steps, "data": "synthetic"}
    print(json.dumps(rec), flush=True)


def study_topk(args):
    """Per-token time at top-k 1, 2, 4 on the fine-grained layer with the
    shared expert (the MXFP4 layer's architecture, T = 16384)."""
    import numpy as np
    import torch

    from mixture_experts_layer_25_amd import moe, synthetic as syn, upload

    base = syn.CONFIGS["fine384_mxfp4"]
    inp = syn.make_inputs(base)
    c0, x, W_r, bias, w = upload.to_device(inp)
    del inp
    stream = torch.cuda.current_stream()
    wstruct = w.struct()
    for k in (1, 2, 4):
        c = moe.make_cfg(T=base.T, D=base.D, E=base.E, F=base.F, top_k=k, gating=base.gating,
                         renorm=bool(base.renorm), capacity=base.capacity, clamp=base.clamp,
                         act=base.act, w=base.wdt, shared_F=base.shared_F)
        ws = moe.workspace(c, moe.WS_FORWARD, x.device)
        y = torch.empty((base.T, base.D), dtype=torch.bfloat16, device=x.device)
        idx = torch.empty((base.T, k), dtype=torch.int32, device=x.device)
        tw = torch.empty((base.T, k), dtype=torch.float32, device=x.device)
        counts = torch.empty(base.E, dtype=torch.int32, device=x.device)
        offsets = torch.empty(base.E + 1, dtype=torch.int32, device=x.device)

        def fwd():
            moe.forward(c, x, W_r, bias, w, y=y, ws=ws, topk_idx=idx, topk_w=tw, counts=counts,
                        offsets=offsets, wstruct=wstruct)
        steps, _ = _time_steps([fwd], args.steps, args.warmup, stream)
        per_tok_us = [1e3 * ms / base.T for ms in steps]
        kept = int(offsets[-1].item())
        # the shared expert is added once: y(with) - y(without) against its own output
        c_ns = moe.make_cfg(T=base.T, D=base.D, E=base.E, F=base.F, top_k=k, gating=base.gating,
                            renorm=bool(base.renorm), capacity=base.capacity, clamp=base.clamp,
                            act=base.act, w=base.wdt, shared_F=0)
        y_ns = moe.forward(c_ns, x, W_r, bias, w)
        _, y_sh = moe.shared_expert(c, x, w)
        torch.cuda.synchronize()
        diff = (y.float() - y_ns.float()).double()
        sh = y_sh[:base.T].double()
        # least-squares coefficient of y(with) - y(without) on the shared
        # output: 1 when it is added once, 2 if it were added twice
        scale = float((diff * sh).sum() / (sh * sh).sum())
        # residual against two bf16 roundings of the outputs
        lim = 2e-2 * torch.clamp(sh.abs(), min=1.0) + 2.0 ** -7 * y.double().abs()
        within = bool(((diff - sh).abs() <= lim).all())
        rec = {"study": "topk_sweep", "layer": "fine384_mxfp4 architecture, T=16384, shared expert",
               "top_k": k, "ms_per_step_mean": round(float(np.mean(steps)), 4),
               "per_token_us": {"p50": round(pct(per_tok_us, 50), 5), "p95": round(pct(per_tok_us, 95), 5),
                                "p99": round(pct(per_tok_us, 99), 5)},
               "kept_pairs": kept, "top_misses": base.T * k - kept,
               "shared_output_coefficient": round(scale, 6), "shared_within_rounding": within,
               "steps": args.steps, "data": "synthetic"}
        print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.study:
        if args.gpus != 1:
            print("the studies run on one GPU", file=sys.stderr)
            sys.exit(2)
        return study_dense_vs_moe(args) if args.study == "dense-vs-moe" else study_topk(args)
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace, args.workload, args.profile_command)
    if args.summarize_pmc:
        return summarize_pmc(*args.summarize_pmc, args.workload, args.profile_command)
    if args.summarize_mfma:
        return summarize_mfma(args.summarize_mfma, args.workload, args.profile_command)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures the layer on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the multi-GPU sharding is design-only.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mixture_experts_layer_25_amd import moe, synthetic as syn, upload

    cfg = syn.CONFIGS[args.workload]
    t_gen = time.time()
    inp = syn.make_inputs(cfg)
    log(f"[bench] generated {cfg.name} inputs in {time.time() - t_gen:.1f}s")
    c, x, W_r, bias, w = upload.to_device(inp)
    del inp
    dev = x.device
    wstruct = w.struct()
    L = moe.lib()
    T, k, E = cfg.T, cfg.k, cfg.E
    ws = moe.workspace(c, moe.WS_FORWARD, dev)
    y = torch.empty((T, cfg.D), dtype=moe.act_torch_dtype(c), device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)

    def fwd():
        moe.forward(c, x, W_r, bias, w, y=y, ws=ws, topk_idx=idx, topk_w=tw, counts=counts,
                    offsets=offsets, wstruct=wstruct)

    # The timed steps are moe_forward itself. A second pass runs the layer
    # through its stage entry points (the same kernels moe_forward launches,
    # in the same order, on the same stream, the gate/up GEMM gathering its
    # rows from x as in moe_forward), with a HIP event between stages, so
    # that each stage's duration is known.
    d_ws = moe.workspace(c, moe.WS_DISPATCH, dev)
    f_ws = moe.workspace(c, moe.WS_EXPERT_FFN, dev)
    r_ws = moe.workspace(c, moe.WS_ROUTE, dev)
    tk = T * k
    slot_pos = torch.empty((T, k), dtype=torch.int32, device=dev)
    perm = torch.empty(tk, dtype=torch.int32, device=dev)
    # bf16 activations: as in moe_forward, dispatch copies no rows and the
    # gate/up GEMM gathers them from x through perm
    gathered = cfg.act == syn.BF16
    x_perm = None if gathered else torch.empty((tk, cfg.D), dtype=moe.act_torch_dtype(c), device=dev)
    H = torch.empty((tk, cfg.F), dtype=moe.act_torch_dtype(c), device=dev)
    y_perm = torch.empty((tk, cfg.D), dtype=torch.float32, device=dev)
    Hs = ys = None
    if cfg.shared_F:
        Hs = torch.empty((T, cfg.shared_F), dtype=torch.bfloat16, device=dev)
        ys = torch.empty((T, cfg.D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    import ctypes
    P = ctypes.byref
    sp = moe._stream(stream)

    stages = {
        # the router moe_forward runs (screened for many experts)
        "route": lambda: L.moe_route_screened(P(c), x.data_ptr(), W_r.data_ptr(),
                                              bias.data_ptr() if bias is not None else None,
                                              idx.data_ptr(), tw.data_ptr(), r_ws.data_ptr(),
                                              r_ws.numel(), sp),
        "dispatch": lambda: L.moe_dispatch(P(c), idx.data_ptr(), x.data_ptr(), counts.data_ptr(),
                                           offsets.data_ptr(), slot_pos.data_ptr(),
                                           perm.data_ptr(),
                                           None if gathered else x_perm.data_ptr(),
                                           d_ws.data_ptr(), d_ws.numel(), sp),
        "gate_up": (lambda: L.moe_expert_gate_up_gathered(
                        P(c), x.data_ptr(), perm.data_ptr(), offsets.data_ptr(), P(wstruct),
                        H.data_ptr(), f_ws.data_ptr(), f_ws.numel(), sp)) if gathered else
                   (lambda: L.moe_expert_gate_up(P(c), x_perm.data_ptr(), offsets.data_ptr(),
                                                 P(wstruct), H.data_ptr(), f_ws.data_ptr(),
                                                 f_ws.numel(), sp)),
        "down": lambda: L.moe_expert_down(P(c), H.data_ptr(), offsets.data_ptr(), P(wstruct),
                                          y_perm.data_ptr(), f_ws.data_ptr(), f_ws.numel(), sp),
        "combine": lambda: L.moe_combine(P(c), y_perm.data_ptr(), slot_pos.data_ptr(),
                                         tw.data_ptr(), ys.data_ptr() if ys is not None else None,
                                         y.data_ptr(), sp),
    }
    if cfg.shared_F:
        stages["shared"] = lambda: L.moe_shared_expert(P(c), x.data_ptr(), P(wstruct),
                                                       Hs.data_ptr(), ys.data_ptr(), sp)
        order = ["route", "dispatch", "gate_up", "down", "shared", "combine"]
    else:
        order = ["route", "dispatch", "gate_up", "down", "combine"]
    fns = [stages[n] for n in order]

    def step(evs=None):
        if evs is not None:
            evs[0].record(stream)
        for i, fn in enumerate(fns):
            rc = fn()
            if rc != 0:
                raise moe.MoEError(rc, f"{order[i]}: status {rc}")
            if evs is not None:
                evs[i + 1].record(stream)

    def new_event():
        return torch.cuda.Event(enable_timing=True)

    # ---------------- whole-layer timing: K steps of moe_forward
    for _ in range(args.warmup):
        fwd()
    fev = [(new_event(), new_event()) for _ in range(args.steps)]
    all0, all1 = new_event(), new_event()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    all0.record(stream)
    for e0, e1 in fev:
        e0.record(stream)
        fwd()
        e1.record(stream)
    all1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = all0.elapsed_time(all1)
    ms_step = ms_total / args.steps
    per_step = [e0.elapsed_time(e1) for e0, e1 in fev]
    A = int(offsets[-1].item())
    cnt = counts.cpu().numpy()
    log(f"[bench] {args.steps} steps of moe_forward: {ms_step:.3f} ms/step "
        f"(wall {wall * 1e3 / args.steps:.3f}), kept pairs {A}, per-expert counts "
        f"{cnt.min()}..{cnt.max()}")

    # ---------------- stage breakdown: K steps through the stage entry points
    for _ in range(max(1, args.warmup // 2)):
        step()
    ev = [[new_event() for _ in range(len(order) + 1)] for _ in range(args.steps)]
    s0, s1 = new_event(), new_event()
    torch.cuda.synchronize()
    s0.record(stream)
    for evs in ev:
        step(evs)
    s1.record(stream)
    torch.cuda.synchronize()
    stagewise_ms = s0.elapsed_time(s1) / args.steps
    stage_roof = [evs[order.index("gate_up")].elapsed_time(evs[order.index("gate_up") + 1])
                  for evs in ev]
    stage_ms = {n: sum(evs[i].elapsed_time(evs[i + 1]) for evs in ev) / args.steps
                for i, n in enumerate(order)}
    log(f"[bench] stage by stage: {stagewise_ms:.3f} ms/step")

    # ---------------- memory-bound stages with the MALL flushed: before each
    # stage a 512 MiB read (twice the 256 MB Infinity Cache) evicts what the
    # previous stage left there; the stage is timed alone. A read rather
    # than a write, so that the cache is left holding clean lines and the
    # timed stage does not also pay for writing a flush buffer back.
    flush = torch.ones(128 * 1024 * 1024, dtype=torch.int32, device=dev)
    nfl = min(args.steps, 10)
    mem_bound = ("route", "dispatch", "combine")
    fl_ms = {n: 0.0 for n in mem_bound}
    for _ in range(nfl):
        for n, fn in zip(order, fns):
            if n not in mem_bound:
                continue
            flush.max()
            a0, a1 = new_event(), new_event()
            a0.record(stream)
            rc = fn()
            a1.record(stream)
            if rc != 0:
                raise moe.MoEError(rc, f"{n}: status {rc}")
            torch.cuda.synchronize()
            fl_ms[n] += a0.elapsed_time(a1) / nfl
    del flush
    work = algorithmic(cfg, A)

    if args.copy_calibration:
        src = torch.empty(256 * 1024 * 1024, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def tfs(flop, ms):
        return flop / (ms * 1e-3) / 1e12

    def gbs(b, ms):
        return b / (ms * 1e-3) / 1e9

    gu_tf = tfs(work["gate_up_flop"], stage_ms["gate_up"])
    dn_tf = tfs(work["down_flop"], stage_ms["down"])
    gemm_tf = tfs(work["gate_up_flop"] + work["down_flop"], stage_ms["gate_up"] + stage_ms["down"])
    stage_report = {
        "route": {"ms": stage_ms["route"], "GB/s": gbs(work["route_bytes"], stage_ms["route"])},
        "dispatch": {"ms": stage_ms["dispatch"], "GB/s": gbs(work["dispatch_bytes"], stage_ms["dispatch"]),
                     "bytes": work["dispatch_bytes"],
                     "note": ("index work only (counts, offsets, ranks): the gate/up GEMM gathers "
                              "the rows from x, so no row is copied" if gathered else
                              "indices and the row copy into x_perm")},
        "gate_up": {"ms": stage_ms["gate_up"], "TFLOP/s": gu_tf},
        "down": {"ms": stage_ms["down"], "TFLOP/s": dn_tf},
        "combine": {"ms": stage_ms["combine"], "GB/s": gbs(work["combine_bytes"], stage_ms["combine"])},
    }
    if cfg.shared_F:
        stage_report["shared"] = {"ms": stage_ms["shared"],
                                  "TFLOP/s": tfs(work["shared_flop"], stage_ms["shared"])}
    flushed = {n: {"ms": fl_ms[n], "GB/s": gbs(work[f"{n}_bytes"], fl_ms[n])}
               for n in ("route", "dispatch", "combine")}
    for n in order:
        log(f"[bench] {n:9s} " + "  ".join(f"{kk} {vv:9.3f}" for kk, vv in stage_report[n].items()
                                           if kk in ("ms", "GB/s", "TFLOP/s")))
    log(f"[bench] grouped GEMM {gemm_tf:.1f} TFLOP/s = "
        f"{100 * gemm_tf / PEAK_BF16_TFLOPS:.1f}% of bf16 peak")
    log("[bench] MALL flushed: " + "  ".join(f"{n} {v['ms']:.3f} ms {v['GB/s']:.0f} GB/s"
                                             for n, v in flushed.items()))

    # ---------------- the same forward captured once into a HIP graph and
    # replayed K times (after every other GPU pass: the kernel trace's
    # dispatch order of the first two passes is unchanged, and a failed
    # capture cannot disturb another measurement)
    graph = graph_pass(torch, fwd, stream, args.warmup, args.steps, T)
    if "ms_per_step" in graph:
        log(f"[bench] {args.steps} replays of one captured moe_forward: "
            f"{graph['ms_per_step']:.3f} ms/step")
    else:
        log(f"[bench] graph capture failed: {graph.get('error')}")

    # Roofline of the dominant kernel: the grouped gate/up GEMM with the
    # SwiGLU epilogue. Its duration is the mean of its event intervals inside
    # the timed steps (the interval also holds the tiny tile-map kernel).
    rk = roofline_kernel(cfg)
    traffic = None
    tf_path = TRAFFIC_FILE.format(workload=cfg.name)
    if os.path.exists(tf_path):
        rec = json.load(open(tf_path))
        if rec.get("kernel_src_sha256") == src_sha256(rk["src"]) and rec.get("kernel") == rk["name"]:
            traffic = rec.get("bytes_per_launch")
    if rk["bound"] == "alu":
        peak, unit = PEAK_FP32_TFLOPS, "TFLOP/s"
    else:
        peak, unit = rk.get("peak", PEAK_BF16_TFLOPS), "TFLOP/s"
    roofline = {"bound": rk["bound"], "achieved": gu_tf, "peak": peak, "unit": unit,
                "frac": gu_tf / peak, "traffic": traffic,
                "kernel": rk["name"],
                "algorithmic": f"4*D*F flop per kept (token, expert) pair x {A} pairs = "
                               f"{work['gate_up_flop'] / 1e9:.3f} GFLOP per launch"}

    # ---------------- CPU oracle baseline (bounded sample)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": T * args.steps / (ms_total * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "stagewise_ms_per_step": stagewise_ms,
        "graph_replay": graph,
        "p50_ms": pct(per_step, 50), "p95_ms": pct(per_step, 95), "p99_ms": pct(per_step, 99),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("mxfp8" if cfg.wdt == 3 else "bf16") if cfg.act == 1 else "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: T={T} D={cfg.D} E={E} top-{k} F={cfg.F} "
                               f"{'bf16' if cfg.act == 1 else 'fp32'} act, "
                               f"{['fp32', 'bf16', 'mxfp4', 'mxfp4'][cfg.wdt]} weights"
                               f"{', mxfp8 expert activations' if cfg.wdt == 3 else ''}",
                   "tokens": T, "kept_pairs": A, "seed": 0},
        "grouped_gemm_tflops": gemm_tf,
        "grouped_gemm_frac_of_bf16_peak": gemm_tf / PEAK_BF16_TFLOPS,
        "stages": stage_report,
        "stages_mall_flushed": flushed,
        "env": environment(torch, dev),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def graph_pass(torch, fwd, stream, warmup, steps, T):
    """One moe_forward captured into a HIP graph (torch.cuda.CUDAGraph: the
    binding passes the capture stream as the call's stream), replayed
    `steps` times after `warmup` replays; ms per replay and tokens/s."""
    try:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            fwd()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fwd()
        torch.cuda.synchronize()
        for _ in range(warmup):
            g.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        return {"ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3)}
    except RuntimeError as ex:  # recorded in the JSON line, not hidden
        return {"error": str(ex)[:200]}


def _smi(*args):
    """rocm-smi's JSON answer for one card (empty if the tool is missing)."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", *args, "--json"], capture_output=True, text=True, timeout=30)
        d = json.loads(r.stdout or "{}")
    except Exception:
        return {}
    cards = [v for kk, v in d.items() if kk.startswith("card")]
    return {**(cards[0] if cards else {}), **d.get("system", {})}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def environment(torch, dev):
    """Device, clocks (as rocm-smi reports them after the timed work),
    driver and software versions, host CPU."""
    p = torch.cuda.get_device_properties(dev)
    clocks = _smi("--showclocks")
    drv = _smi("--showdriverversion")
    return {"device": torch.cuda.get_device_name(dev), "arch": getattr(p, "gcnArchName", ""),
            "cus": p.multi_processor_count, "hip": torch.version.hip, "torch": torch.__version__,
            "gpu_clocks": {kk: v for kk, v in clocks.items() if "clock" in kk.lower()},
            "driver": {kk: v for kk, v in drv.items() if "driver" in kk.lower()},
            "host_cpu": cpu_model(), "host_threads": os.cpu_count()}


def _tiny_single_thread():
    """The oracle on the whole tiny fp32 layer (T = 64) with one thread, in a
    child process (its OpenMP runtime then starts with one thread)."""
    import subprocess
    code = ("import time, oracle; from mixture_experts_layer_25_amd import synthetic as syn; "
            "inp = syn.make_inputs(syn.CONFIGS['tiny_fp32']); oracle.forward(inp); "
            "t = time.perf_counter(); [oracle.forward(inp) for _ in range(5)]; "
            "print((time.perf_counter() - t) / 5)")
    env = {**os.environ, "OMP_NUM_THREADS": "1"}
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=300)
    s = float(r.stdout.strip().splitlines()[-1])
    return {"value": 64 / s, "unit": "tokens/s", "cores": 1, "seconds_per_layer": s,
            "sample": "the whole tiny_fp32 layer (T=64, D=128, E=8, top-2, F=256), "
                      "mean of 5 runs"}


def cpu_baseline(cfg, seconds):
    """The CPU oracle, as it stands, on the first n tokens of the same
    workload treated as a layer of n tokens (route, dispatch, experts,
    combine). n is sized from a short calibration run to about `seconds`."""
    import numpy as np

    import oracle
    from mixture_experts_layer_25_amd import synthetic as syn

    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or (os.cpu_count() or 1)
    full = syn.make_inputs(cfg)

    def run(n):
        sub = syn.Inputs(**{**full.__dict__})
        sub.cfg = cfg.replace(T=n, capacity=cfg.capacity)
        sub.x = np.ascontiguousarray(full.x[:n])
        t = time.perf_counter()
        oracle.forward(sub)
        return time.perf_counter() - t

    n0 = max(1, min(cfg.T, threads))
    t0 = run(n0)
    n = int(min(cfg.T, max(n0, n0 * max(1.0, seconds / max(t0, 1e-3)))))
    n = max(n0, (n // n0) * n0)
    t = run(n) if n != n0 else t0
    log(f"[bench] cpu oracle: {n} tokens in {t:.2f}s on {threads} threads")
    single = _tiny_single_thread()
    log(f"[bench] cpu oracle, tiny fp32 layer, one thread: {single['value']:.0f} tokens/s")
    return {"value": n / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"first {n} tokens of the {cfg.name} workload as an {n}-token layer "
                      f"(full route, dispatch, {cfg.k} SwiGLU experts per token, combine)",
            "tiny_fp32_one_thread": single}


if __name__ == "__main__":
    main()
