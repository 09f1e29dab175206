"""moe_dispatch_noalloc (the library's fixed device scratch instead of a
caller's workspace) against moe_dispatch on the same inputs: two calls in a
row, the second with a smaller layer, every output bit-exact; and a layer
beyond the scratch is rejected before anything is enqueued."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_25_amd import moe, synthetic as syn, upload

pytestmark = pytest.mark.gpu


def _outs(cfg, dev):
    tk = max(cfg.T * cfg.k, 1)
    return dict(counts=torch.full((cfg.E,), -7, dtype=torch.int32, device=dev),
                offsets=torch.full((cfg.E + 1,), -7, dtype=torch.int32, device=dev),
                slot_pos=torch.full((cfg.T, cfg.k), -7, dtype=torch.int32, device=dev),
                perm=torch.full((tk,), -1, dtype=torch.int32, device=dev),
                x_perm=torch.zeros((tk, cfg.D), dtype=torch.bfloat16, device=dev))


def _check_case(cfg):
    print(f"[noalloc] {cfg}", flush=True)
    inp = syn.make_inputs(cfg, with_experts=False)
    c = upload.cfg_of(cfg)
    x = upload._dev_bits(inp.x, "cuda")
    W_r = upload._dev_bits(inp.W_r, "cuda")
    bias = upload._dev_bits(inp.bias, "cuda") if inp.bias is not None else None
    idx, _, _ = moe.route(c, x, W_r, bias)
    ref = moe.dispatch(c, idx, x)
    got = _outs(cfg, x.device)
    moe.dispatch_noalloc(c, idx, x, got["counts"], got["offsets"], got["slot_pos"], got["perm"],
                         got["x_perm"])
    torch.cuda.synchronize()
    A = int(ref["offsets"][-1].item())
    for k in ("counts", "offsets", "slot_pos"):
        assert torch.equal(got[k], ref[k]), k
    assert torch.equal(got["perm"][:A], ref["perm"][:A])
    assert torch.equal(got["x_perm"][:A].view(torch.int16), ref["x_perm"][:A].view(torch.int16))
    return A


def test_noalloc_dispatch_matches_workspace_dispatch_twice():
    big = syn.Config("noalloc_big", T=5000, D=256, E=128, k=8, F=64, bias="normal",
                     bias_sigma=1.0, capacity=300)
    small = syn.Config("noalloc_small", T=700, D=128, E=24, k=3, F=64, bias="normal",
                       bias_sigma=0.5)
    a1 = _check_case(big)
    a2 = _check_case(small)
    assert a1 > 0 and a2 > 0


def test_noalloc_dispatch_rejects_beyond_scratch():
    # E * ceil(T/256) = 1024 * 257 > 262144 int32 entries
    cfg = syn.Config("noalloc_over", T=256 * 257, D=64, E=1024, k=1, F=64)
    c = upload.cfg_of(cfg)
    d = torch.zeros(16, dtype=torch.int32, device="cuda")
    with pytest.raises(moe.MoEError) as ei:
        moe.dispatch_noalloc(c, d, d, d, d, d, d, d)
    assert ei.value.status == -5
