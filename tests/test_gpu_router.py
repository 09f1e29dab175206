"""Every router kernel instance against the oracle: expert counts in each
range the launcher distinguishes (<= 8, <= 16, 17-32, 33-64, 65-128,
129-256, 257-384, 385-512, 513-1024), the 8-expert kernel beyond its
width limit (D = 8192 falls back to the general few-expert kernel), and
top_k up to the ABI's limit of 16. Indices and logits bit-exact (one fp32
FMA chain per logit on both sides), weights within 1e-5."""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_25_amd import moe, synthetic as syn, upload

pytestmark = pytest.mark.gpu

CASES = [
    # (E, k, D, gating, renorm, x dtype)
    (8, 2, 8192, syn.GATE_SOFTMAX, 1, syn.BF16),
    (8, 8, 8192, syn.GATE_SQRT_SOFTPLUS, 0, syn.F32),
    (5, 3, 256, syn.GATE_SIGMOID, 1, syn.BF16),
    (16, 16, 512, syn.GATE_SOFTMAX, 1, syn.BF16),
    (24, 7, 512, syn.GATE_SIGMOID, 0, syn.BF16),
    (32, 16, 512, syn.GATE_SOFTMAX, 0, syn.F32),
    (64, 16, 512, syn.GATE_SQRT_SOFTPLUS, 0, syn.BF16),
    (100, 9, 512, syn.GATE_SOFTMAX, 1, syn.BF16),
    (256, 8, 512, syn.GATE_SOFTMAX, 1, syn.BF16),
    (200, 16, 256, syn.GATE_SIGMOID, 1, syn.F32),
    (384, 16, 512, syn.GATE_SQRT_SOFTPLUS, 0, syn.BF16),
    (512, 6, 512, syn.GATE_SOFTMAX, 1, syn.BF16),
    (450, 12, 256, syn.GATE_SQRT_SOFTPLUS, 0, syn.F32),
    (1024, 16, 512, syn.GATE_SOFTMAX, 1, syn.BF16),
    (700, 8, 256, syn.GATE_SIGMOID, 0, syn.BF16),
]


@pytest.mark.parametrize("E,k,D,gating,renorm,act", CASES)
def test_router_instance(E, k, D, gating, renorm, act):
    wdt = syn.F32 if act == syn.F32 else syn.BF16
    cfg = syn.Config(f"router_E{E}_k{k}", T=301, D=D, E=E, k=k, F=64, act=act, wdt=wdt,
                     gating=gating, renorm=renorm, bias="normal", bias_sigma=0.3)
    print(f"[router] {cfg}", flush=True)
    inp = syn.make_inputs(cfg, with_experts=False)
    logits, idx, w = oracle.route(cfg, inp.x, inp.W_r, inp.bias)
    c = upload.cfg_of(cfg)
    x = upload._dev_bits(inp.x, "cuda")
    W_r = upload._dev_bits(inp.W_r, "cuda")
    bias = upload._dev_bits(inp.bias, "cuda")
    gi, gw, gl = moe.route(c, x, W_r, bias, want_logits=True)
    torch.cuda.synchronize()
    assert np.array_equal(gl.cpu().numpy().view(np.uint32), logits.view(np.uint32)), \
        "logits not bit-identical"
    assert np.array_equal(gi.cpu().numpy(), idx), "expert indices differ"
    gw = gw.cpu().numpy()
    assert np.allclose(gw, w, rtol=1e-5, atol=1e-6), f"weights: max diff {np.abs(gw - w).max():.3g}"
    # without the optional logits output the same selection and weights
    gi2, gw2, _ = moe.route(c, x, W_r, bias)
    torch.cuda.synchronize()
    assert np.array_equal(gi2.cpu().numpy(), idx)
    assert np.array_equal(gw2.cpu().numpy().view(np.uint32), gw.view(np.uint32))


SCREEN_CASES = [
    # (E, k, D, gating, renorm); the screen runs from 128 experts, below
    # that the entry point runs the exact router
    (64, 4, 512, syn.GATE_SOFTMAX, 1),
    (128, 8, 1024, syn.GATE_SOFTMAX, 1),
    (200, 8, 512, syn.GATE_SIGMOID, 1),
    (256, 8, 512, syn.GATE_SIGMOID, 1),
    (256, 16, 256, syn.GATE_SIGMOID, 0),
    (300, 9, 512, syn.GATE_SQRT_SOFTPLUS, 0),
    (384, 6, 1024, syn.GATE_SQRT_SOFTPLUS, 0),
    (512, 16, 256, syn.GATE_SOFTMAX, 1),
    (1024, 6, 512, syn.GATE_SQRT_SOFTPLUS, 0),
    (260, 5, 4096, syn.GATE_SOFTMAX, 1),
    # softmax without renormalisation: the screened entry runs the exact router
    (384, 4, 256, syn.GATE_SOFTMAX, 0),
]


def _route_both(cfg, inp):
    c = upload.cfg_of(cfg)
    x = upload._dev_bits(inp.x, "cuda")
    W_r = upload._dev_bits(inp.W_r, "cuda")
    bias = upload._dev_bits(inp.bias, "cuda") if inp.bias is not None else None
    ei, ew, _ = moe.route(c, x, W_r, bias)
    si, sw = moe.route_screened(c, x, W_r, bias)
    torch.cuda.synchronize()
    return ei.cpu().numpy(), ew.cpu().numpy(), si.cpu().numpy(), sw.cpu().numpy()


@pytest.mark.parametrize("E,k,D,gating,renorm", SCREEN_CASES)
def test_screened_router_equals_exact(E, k, D, gating, renorm):
    """moe_route_screened (MFMA estimate, candidates within the error bound,
    exact chains for those only) writes the same indices and the same weight
    bits as the exact router, and the indices equal the oracle's."""
    cfg = syn.Config(f"screen_E{E}", T=777, D=D, E=E, k=k, F=64, gating=gating, renorm=renorm,
                     bias="normal", bias_sigma=0.3)
    print(f"[router] screened {cfg}", flush=True)
    inp = syn.make_inputs(cfg, with_experts=False)
    ei, ew, si, sw = _route_both(cfg, inp)
    _, idx, w = oracle.route(cfg, inp.x, inp.W_r, inp.bias)
    assert np.array_equal(si, idx), "screened indices differ from the oracle"
    assert np.array_equal(si, ei)
    assert np.array_equal(sw.view(np.uint32), ew.view(np.uint32)), "weights not bit-identical"


def test_screened_router_ties_and_zero_rows():
    """All-tie tokens (zero rows without a bias: every expert is a candidate,
    several passes of exact chains), duplicated W_r columns (exact ties,
    decided toward the lower index) and scaled rows."""
    E, k, D, T = 320, 6, 512, 300
    cfg = syn.Config("screen_ties", T=T, D=D, E=E, k=k, F=64, gating=syn.GATE_SQRT_SOFTPLUS,
                     renorm=0)
    inp = syn.make_inputs(cfg, with_experts=False)
    x = syn.bf16_bits_to_f32(inp.x).copy()
    x[::7] = 0.0                     # zero rows
    x[3::11] *= 40.0                 # large rows
    inp.x = syn.f32_to_bf16_bits(x)
    inp.W_r[:, 50] = inp.W_r[:, 10]  # duplicated experts
    inp.W_r[:, 151] = inp.W_r[:, 150]
    ei, ew, si, sw = _route_both(cfg, inp)
    _, idx, w = oracle.route(cfg, inp.x, inp.W_r, inp.bias)
    assert np.array_equal(si, idx)
    assert np.array_equal(si, ei)
    assert np.array_equal(sw.view(np.uint32), ew.view(np.uint32))
    assert (idx[::7] == np.arange(k)).all()   # zero rows: the lowest indices
