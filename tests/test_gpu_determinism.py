"""Repeated runs give bit-identical results.

The grouped GEMMs split the tiles of their last round along K and add the
parts' partial sums in a fixed order, and the router and dispatch are
integer or fixed-order work, so the whole layer must be reproducible bit for
bit. A data race (an LDS hand-off, a flag, a register read too early) shows
up here as differences between runs even when every run is within the
oracle's tolerance."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_25_amd import moe, synthetic as syn, upload
from split_cases import SPLIT_CASES

pytestmark = pytest.mark.gpu

CASES = {
    # small shapes (K < 2048: no tile is split along K)
    "mixtral_small": syn.small_variant(syn.CONFIGS["mixtral"], T=300, D=256, F=352),
    "fine384_small": syn.small_variant(syn.CONFIGS["fine384_mxfp4"], T=200, D=256, F=128),
    "capacity_small": syn.small_variant(syn.CONFIGS["capacity"], T=500, D=256, F=160),
    "fine384_a8_small": syn.small_variant(syn.CONFIGS["fine384_mxfp4_a8"], T=200, D=256, F=128),
    # full Mixtral shape: the down GEMM's last round is split 4 ways
    "mixtral": syn.CONFIGS["mixtral"],
}
# small shapes whose tiles are split along K in 2, 4 and 8 parts (the host
# replica of the schedule checks that they split)
CASES.update({n: c for n, (c, _) in SPLIT_CASES.items()})


@pytest.mark.parametrize("name", list(CASES))
def test_forward_is_bit_reproducible(name):
    cfg = CASES[name]
    print(f"[determinism] {name}: T={cfg.T} D={cfg.D} E={cfg.E} F={cfg.F}", flush=True)
    inp = syn.make_inputs(cfg)
    c, x, W_r, bias, w = upload.to_device(inp)
    ws = moe.workspace(c, moe.WS_FORWARD, x.device)
    outs = []
    for _ in range(3):
        y = moe.forward(c, x, W_r, bias, w, ws=ws)
        torch.cuda.synchronize()
        outs.append(upload.to_host_bits(y))
    for r in range(1, len(outs)):
        diff = int((outs[r] != outs[0]).sum())
        assert diff == 0, f"{name}: run {r} differs from run 0 in {diff} of {outs[0].size} outputs"
