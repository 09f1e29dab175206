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
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s (1 GPU) + grouped-GEMM TFLOP/s as % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_MXFP4_TFLOPS = 10100.0  # MI355X dense fp4 MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_{workload}.json")
GEMM_SRC = os.path.join(ROOT, "mixture_experts_layer_25_amd", "csrc", "gemm.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral")
    ap.add_argument("--stage-reps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device copy (for counter scaling)")
    return ap.parse_args()


def algorithmic(cfg, A):
    """Algorithmic work of one forward (what the method must compute/move)."""
    sx = 2 if cfg.act == 1 else 4
    T, D, E, k, F = cfg.T, cfg.D, cfg.E, cfg.k, cfg.F
    return dict(
        gate_up_flop=4.0 * D * F * A,
        down_flop=2.0 * D * F * A,
        shared_flop=6.0 * D * cfg.shared_F * T,
        route_bytes=T * D * sx + D * E * 4 + T * k * 8,
        dispatch_bytes=T * k * 8 + T * D * sx + A * D * sx + A * 4,
        combine_bytes=A * D * 4 + T * k * 8 + T * D * sx + (T * D * 4 if cfg.shared_F else 0),
    )


def pct(vals, q):
    v = sorted(vals)
    i = min(len(v) - 1, max(0, int(round(q / 100.0 * (len(v) - 1)))))
    return v[i]


def main():
    args = parse()
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

    # ---------------- whole-layer timing
    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    all0, all1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    all0.record()
    for s, e in ev:
        s.record()
        fwd()
        e.record()
    all1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = all0.elapsed_time(all1)
    ms_step = ms_total / args.steps
    per_step = [s.elapsed_time(e) for s, e in ev]
    A = int(offsets[-1].item())
    cnt = counts.cpu().numpy()
    log(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step (wall {wall * 1e3 / args.steps:.3f}), "
        f"kept pairs {A}, per-expert counts {cnt.min()}..{cnt.max()}")

    # ---------------- per-stage timing (same inputs, separate launches)
    work = algorithmic(cfg, A)
    d_ws = moe.workspace(c, moe.WS_DISPATCH, dev)
    f_ws = moe.workspace(c, moe.WS_EXPERT_FFN, dev)
    tk = T * k
    slot_pos = torch.empty((T, k), dtype=torch.int32, device=dev)
    perm = torch.empty(tk, dtype=torch.int32, device=dev)
    x_perm = torch.empty((tk, cfg.D), dtype=moe.act_torch_dtype(c), device=dev)
    H = torch.empty((tk, cfg.F), dtype=moe.act_torch_dtype(c), device=dev)
    y_perm = torch.empty((tk, cfg.D), dtype=torch.float32, device=dev)
    Hs = ys = None
    if cfg.shared_F:
        Hs = torch.empty((T, cfg.shared_F), dtype=torch.bfloat16, device=dev)
        ys = torch.empty((T, cfg.D), dtype=torch.float32, device=dev)
    flush = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    import ctypes
    P = ctypes.byref
    sp = moe._stream()

    stages = {
        "route": lambda: L.moe_route(P(c), x.data_ptr(), W_r.data_ptr(),
                                     bias.data_ptr() if bias is not None else None,
                                     idx.data_ptr(), tw.data_ptr(), None, sp),
        "dispatch": lambda: L.moe_dispatch(P(c), idx.data_ptr(), x.data_ptr(), counts.data_ptr(),
                                           offsets.data_ptr(), slot_pos.data_ptr(),
                                           perm.data_ptr(), x_perm.data_ptr(), d_ws.data_ptr(),
                                           d_ws.numel(), sp),
        "gate_up": lambda: L.moe_expert_gate_up(P(c), x_perm.data_ptr(), offsets.data_ptr(),
                                                P(wstruct), H.data_ptr(), f_ws.data_ptr(),
                                                f_ws.numel(), sp),
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
    stage_ms = {}
    for name in order:
        fn = stages[name]
        for _ in range(3):
            assert fn() == 0, name
        torch.cuda.synchronize()
        tot = 0.0
        flushed = name in ("route", "dispatch", "combine")
        for _ in range(args.stage_reps):
            if flushed:
                flush.zero_()   # evict the 256 MB MALL so HBM-bound stages read HBM
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
            assert fn() == 0, name
            e.record(stream)
            e.synchronize()
            tot += s.elapsed_time(e)
        stage_ms[name] = tot / args.stage_reps
    del flush
    torch.cuda.synchronize()

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
    peak = PEAK_BF16_TFLOPS
    stage_report = {
        "route": {"ms": stage_ms["route"], "GB/s": gbs(work["route_bytes"], stage_ms["route"])},
        "dispatch": {"ms": stage_ms["dispatch"], "GB/s": gbs(work["dispatch_bytes"], stage_ms["dispatch"])},
        "gate_up": {"ms": stage_ms["gate_up"], "TFLOP/s": gu_tf},
        "down": {"ms": stage_ms["down"], "TFLOP/s": dn_tf},
        "combine": {"ms": stage_ms["combine"], "GB/s": gbs(work["combine_bytes"], stage_ms["combine"])},
    }
    if cfg.shared_F:
        stage_report["shared"] = {"ms": stage_ms["shared"],
                                  "TFLOP/s": tfs(work["shared_flop"], stage_ms["shared"])}
    for n in order:
        log(f"[bench] {n:9s} " + "  ".join(f"{kk} {vv:9.3f}" for kk, vv in stage_report[n].items()))
    log(f"[bench] grouped GEMM {gemm_tf:.1f} TFLOP/s = {100 * gemm_tf / peak:.1f}% of bf16 peak")

    # HBM traffic of the dominant kernel from the committed counter summary
    traffic = None
    tf_path = TRAFFIC_FILE.format(workload=cfg.name)
    if os.path.exists(tf_path):
        rec = json.load(open(tf_path))
        src_hash = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()
        if rec.get("gemm_src_sha256") == src_hash:
            traffic = rec.get("gate_up_bytes_per_launch")

    roofline = {"bound": "mfma", "achieved": gu_tf, "peak": peak, "unit": "TFLOP/s",
                "frac": gu_tf / peak, "traffic": traffic,
                "kernel": "grouped gate/up GEMM + SwiGLU epilogue (gemm_kernel<SWIGLU>)",
                "algorithmic": f"4*D*F per kept pair x {A} pairs = {work['gate_up_flop'] / 1e9:.1f} GFLOP"}

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
        "p50_ms": pct(per_step, 50), "p95_ms": pct(per_step, 95), "p99_ms": pct(per_step, 99),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.act == 1 else "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: T={T} D={cfg.D} E={E} top-{k} F={cfg.F} "
                               f"{'bf16' if cfg.act == 1 else 'fp32'} act, "
                               f"{['fp32', 'bf16', 'mxfp4'][cfg.wdt]} weights",
                   "tokens": T, "kept_pairs": A, "seed": 0},
        "grouped_gemm_tflops": gemm_tf,
        "grouped_gemm_frac_of_bf16_peak": gemm_tf / peak,
        "stages": stage_report,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


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
    return {"value": n / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} tokens of the {cfg.name} workload as an {n}-token layer "
                      f"(full route, dispatch, {cfg.k} SwiGLU experts per token, combine)"}


if __name__ == "__main__":
    main()
