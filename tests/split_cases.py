"""Small layers whose grouped GEMMs split tiles along K (2, 4 and 8 parts):
few M-tiles and deep K, so that every XCD's round of tiles is partial.
Each case names the K-part count the host replica of the schedule must find
in each GEMM (checked on the CPU by test_tile_plan.py)."""
import numpy as np

import oracle
from mixture_experts_layer_25_amd import synthetic as syn

_BASE = syn.CONFIGS["mixtral"]

SPLIT_CASES = {
    # 8 experts of at most a few hundred rows: gate/up 128 tiles and down
    # 64 (MXFP4 weights: 80 and 40, with wide tails), K = 2048 -> 2 parts
    "split2_bf16": (_BASE.replace(name="split2_bf16", T=300, D=2048, F=2048),
                    {"gate_up": 2, "down": 2}),
    "split2_mxfp4": (_BASE.replace(name="split2_mxfp4", T=300, D=2048, F=2048, wdt=syn.MXFP4),
                     {"gate_up": 2, "down": 2}),
    "split2_a8": (_BASE.replace(name="split2_a8", T=300, D=2048, F=2048, wdt=syn.MXFP4_A8),
                  {"gate_up": 2, "down": 2}),
    # 4 experts of about 60 rows: down 2 tiles per XCD, K = F = 8192 -> 8
    # parts; gate/up K = D = 1024 stays whole
    "split8_down": (_BASE.replace(name="split8_down", T=120, D=1024, E=4, F=8192),
                    {"down": 8}),
    # 4 experts of about 60 rows: down 4 tiles per XCD, K = F = 4096 -> 4
    # parts
    "split4_down": (_BASE.replace(name="split4_down", T=120, D=2048, E=4, F=4096),
                    {"down": 4}),
}


def split_offsets(cfg):
    """Segment offsets of the case's routing (the oracle's)."""
    inp = syn.make_inputs(cfg, with_experts=False)
    _, idx, _ = oracle.route(cfg, inp.x, inp.W_r, inp.bias)
    return oracle.dispatch(cfg, idx)[1]
