"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

Integer results (indices, counts, offsets, slot positions, drops, perm) must
be bit-exact, the router logits bit-identical (one fp32 fused multiply-add
chain per logit on both sides), and y within 1e-4*max(1,|ref|) (fp32 layer)
or 2e-2*max(1,|ref|) (bf16 / MXFP4 layers).
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_25_amd import moe, synthetic as syn, upload
from gpu_helpers import (act_to_f64, assert_close, check_routing, gpu_forward, sample_tokens,
                         stratified_tokens, tol_for)

pytestmark = pytest.mark.gpu

# Small variants of the five workloads: same modes, sizes the oracle finishes
# in seconds, several M- and N-tiles and ragged tails (F, D not multiples of
# the 256/512-column tiles; T not a multiple of 128 rows).
SMALL = {
    "tiny_fp32": syn.CONFIGS["tiny_fp32"],
    "mixtral": syn.small_variant(syn.CONFIGS["mixtral"], T=300, D=256, F=352),
    "capacity": syn.small_variant(syn.CONFIGS["capacity"], T=500, D=256, F=256),
    "fine128": syn.small_variant(syn.CONFIGS["fine128"], T=256, D=256, F=192),
    "fine384_mxfp4": syn.small_variant(syn.CONFIGS["fine384_mxfp4"], T=200, D=256, F=128,
                                       shared_F=96),
    # the same layer with MXFP8 activation operands in the routed experts
    "fine384_mxfp4_a8": syn.small_variant(syn.CONFIGS["fine384_mxfp4_a8"], T=200, D=256, F=128,
                                          shared_F=96),
    # 16 MXFP4 experts of 99..436 rows: full 256-row M-tiles, last M-tiles
    # above 128 rows, and wide last M-tiles of 65..128 and of at most 64 rows
    "mxfp4_mixed_tiles": syn.small_variant(syn.CONFIGS["fine384_mxfp4"], T=600, D=256, F=160,
                                           E=16, shared_F=96),
    # fp32 layer over several 64 x 64 tiles of the fp32 MFMA GEMM: segments
    # of 2-3 M-tiles with ragged last tiles, F and D not multiples of 64,
    # K = D not a multiple of the 16-deep LDS step
    "fp32_tiles": syn.small_variant(syn.CONFIGS["tiny_fp32"], T=300, D=136, F=200),
}


def _oracle_all(inp):
    return oracle.forward(inp)


@pytest.mark.parametrize("name", list(SMALL))
def test_small_stagewise(name):
    cfg = SMALL[name]
    print(f"[parity] small stagewise {name}: {cfg}", flush=True)
    inp = syn.make_inputs(cfg)
    ref = _oracle_all(inp)
    got = gpu_forward(inp, stagewise=True)
    check_routing(cfg, got, ref)
    A = int(ref["offsets"][-1])
    if cfg.wdt == syn.MXFP4_A8:
        # x_perm rows are the MXFP8 quantisation of the x rows of perm_token:
        # codes [T*k][D], then scales grouped as [ceil(D/512)][T*k][16]
        rows, D = cfg.T * cfg.k, cfg.D
        xb = got["x_perm"].reshape(-1).view(np.uint8)
        codes = xb[:rows * D].reshape(rows, D)[:A]
        G = (D + 511) // 512
        sc = xb[rows * D:rows * D + G * rows * 16].reshape(G, rows, 16)
        sc = sc.transpose(1, 0, 2).reshape(rows, G * 16)[:A, :D // 32]
        rc, rs = oracle.mxfp8_quantize(act_to_f64(inp.x[ref["perm"][:A]]))
        assert np.array_equal(sc, rs)
        assert np.array_equal(np.where(codes == 0x80, 0, codes), np.where(rc == 0x80, 0, rc))
    else:
        # x_perm rows are the byte-exact x rows of perm_token
        assert np.array_equal(got["x_perm"][:A], inp.x[ref["perm"][:A]])
    err = assert_close(got["y"], ref["y"], tol_for(cfg), f"{name} y")
    print(f"[parity] {name}: max rel err {err:.3g}", flush=True)


@pytest.mark.parametrize("name", list(SMALL))
def test_small_fused_equals_stagewise(name):
    cfg = SMALL[name]
    inp = syn.make_inputs(cfg)
    a = gpu_forward(inp, stagewise=True)
    b = gpu_forward(inp, stagewise=False)
    assert np.array_equal(a["idx"], b["idx"])
    assert np.array_equal(a["w"].view(np.uint32), b["w"].view(np.uint32))
    assert np.array_equal(a["y"], b["y"]), "fused forward differs from the stage-by-stage calls"
    c = gpu_forward(inp, stagewise=False)
    assert np.array_equal(b["y"], c["y"]), "two runs differ (must be deterministic)"


@pytest.mark.parametrize("name", [n for n in SMALL if SMALL[n].act != syn.F32])
def test_small_gathered_gate_up_equals_dispatched(name):
    """moe_expert_gate_up_gathered (rows read from x through perm_token, after
    a dispatch that copies no rows) writes the same H, byte for byte, as
    moe_expert_gate_up on the dispatched copy x_perm."""
    cfg = SMALL[name]
    inp = syn.make_inputs(cfg)
    c, x, W_r, bias, w = upload.to_device(inp)
    idx, _, _ = moe.route(c, x, W_r, bias)
    d = moe.dispatch(c, idx, x)
    g = moe.dispatch(c, idx, x, copy_rows=False)
    ws = moe.workspace(c, moe.WS_EXPERT_FFN, x.device)
    rows = cfg.T * cfg.k
    H1 = torch.zeros((rows, cfg.F), dtype=torch.bfloat16, device=x.device)
    H2 = torch.zeros_like(H1)
    moe.expert_gate_up(c, d["x_perm"], d["offsets"], w, H1, ws)
    moe.expert_gate_up_gathered(c, x, g["perm"], g["offsets"], w, H2, ws)
    torch.cuda.synchronize()
    for k in ("counts", "offsets", "slot_pos", "perm"):
        assert torch.equal(d[k], g[k]), k
    assert torch.equal(H1.view(torch.int16), H2.view(torch.int16)), "gathered gate/up differs"


@pytest.mark.timeout(400)
@pytest.mark.parametrize("name", syn.CONFIG_ORDER + ["fine384_mxfp4_a8"])
def test_full_size(name):
    """Full workload, in the launch configuration the benchmark times:
    routing on every token; dispatch (counts, offsets, slot positions with
    the drop decisions, perm_token) bit for bit on every pair, from a
    full-size moe_dispatch of the forward's own indices; y on a sample of
    tokens that covers every expert and a row of every M-tile with a tile
    split along K."""
    cfg = syn.CONFIGS[name]
    print(f"[parity] full {name}: generating", flush=True)
    inp = syn.make_inputs(cfg)
    print(f"[parity] full {name}: gpu", flush=True)
    c, x, W_r, bias, w = upload.to_device(inp)
    dev = x.device
    idx_d = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
    tw_d = torch.empty(idx_d.shape, dtype=torch.float32, device=dev)
    cnt_d = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    off_d = torch.empty(cfg.E + 1, dtype=torch.int32, device=dev)
    y = moe.forward(c, x, W_r, bias, w, topk_idx=idx_d, topk_w=tw_d, counts=cnt_d,
                    offsets=off_d)
    d = moe.dispatch(c, idx_d, x)
    torch.cuda.synchronize()
    got = dict(idx=idx_d.cpu().numpy(), w=tw_d.cpu().numpy(), counts=cnt_d.cpu().numpy(),
               offsets=off_d.cpu().numpy(), slot_pos=d["slot_pos"].cpu().numpy(),
               perm=d["perm"].cpu().numpy(), y=upload.to_host_bits(y)[:cfg.T])
    del d, y
    print(f"[parity] full {name}: oracle routing", flush=True)
    logits, idx, w_ref = oracle.route(cfg, inp.x, inp.W_r, inp.bias)
    counts, offsets, slot_pos, perm = oracle.dispatch(cfg, idx)
    ref = dict(idx=idx, w=w_ref, counts=counts, offsets=offsets, slot_pos=slot_pos, perm=perm)
    check_routing(cfg, got, ref)
    n_drop = int((slot_pos < 0).sum())
    if cfg.capacity > 0:
        assert n_drop > 0, "capacity workload should drop pairs"
    toks = stratified_tokens(cfg, idx, slot_pos, perm, offsets, n=32 if cfg.T > 64 else cfg.T)
    print(f"[parity] full {name}: {n_drop} drops bit-exact; oracle y on {len(toks)} tokens",
          flush=True)
    y_exact, y_ref = oracle.forward_tokens(inp, idx, w_ref, slot_pos, toks)
    err = assert_close(got["y"][toks], y_ref, tol_for(cfg), f"{name} y")
    print(f"[parity] full {name}: counts min {counts.min()} max {counts.max()} "
          f"kept {offsets[-1]} of {cfg.T * cfg.k}; max rel err {err:.3g}", flush=True)


def test_dense_gemm_path_vs_torch_matmul():
    """The dense launch (one segment of all rows, used by the shared expert)
    against torch matmuls in float32 on the CPU: H = SiLU(x Wg) * (x Wu)
    rounded to bf16, y = H Wd."""
    cfg = syn.Config("dense", T=333, D=512, E=1, k=1, F=64, shared_F=416, clamp=0.0)
    inp = syn.make_inputs(cfg)
    c, x, W_r, bias, w = upload.to_device(inp)
    H, y = moe.shared_expert(c, x, w)
    torch.cuda.synchronize()
    xf = torch.from_numpy(syn.bf16_bits_to_f32(inp.x))
    Wg = torch.from_numpy(syn.bf16_bits_to_f32(inp.Ws_gate))
    Wu = torch.from_numpy(syn.bf16_bits_to_f32(inp.Ws_up))
    Wd = torch.from_numpy(syn.bf16_bits_to_f32(inp.Ws_down))
    g = xf @ Wg
    u = xf @ Wu
    h = (torch.nn.functional.silu(g) * u).to(torch.bfloat16)
    href = h.float().numpy()
    hgot = H.float().cpu().numpy()
    assert np.abs(hgot - href).max() <= 2 ** -7 * np.abs(href).max() + 1e-6
    frac = np.mean(hgot != href)
    assert frac < 2e-3, f"{frac:.2e} of H differ from the bf16-rounded torch value"
    yref = (h.float() @ Wd).numpy()
    ygot = y.cpu().numpy()
    assert np.all(np.abs(ygot - yref) <= 2e-2 * np.maximum(1.0, np.abs(yref)))
    assert np.abs(ygot - yref).max() < 1e-3 * np.abs(yref).max() + 1e-3
