"""Grouped-GEMM tiles split along K (2, 4 and 8 parts): all-token parity
against the oracle, and the give-up path of the split hand-off.

The shapes come from split_cases.py; before any GPU work each test checks
with the host replica of the tile schedule (tile_plan.py) that the GEMMs
really split."""
import numpy as np
import pytest
import torch

import oracle
import tile_plan as tp
from split_cases import SPLIT_CASES
from mixture_experts_layer_25_amd import moe, synthetic as syn, upload
from gpu_helpers import assert_close, check_routing, gpu_forward, tol_for

pytestmark = pytest.mark.gpu


def _wide(cfg):
    """Wide tiles run with MXFP4 weights."""
    return syn.is_mx(cfg.wdt)


def _plan_S(cfg, offsets, gemm):
    swiglu = gemm == "gate_up"
    K, N = (cfg.D, cfg.F) if swiglu else (cfg.F, cfg.D)
    return {t.S for t in tp.plan(offsets, K, N, swiglu, wide=_wide(cfg))}


@pytest.mark.parametrize("name", list(SPLIT_CASES))
def test_split_tiles_all_tokens(name):
    cfg, want = SPLIT_CASES[name]
    print(f"[split] parity {name}: {cfg}", flush=True)
    inp = syn.make_inputs(cfg)
    ref = oracle.forward(inp)
    for gemm, S in want.items():
        assert S in _plan_S(cfg, ref["offsets"], gemm), (gemm, S)
    got = gpu_forward(inp, stagewise=True)
    check_routing(cfg, got, ref)
    err = assert_close(got["y"], ref["y"], tol_for(cfg), f"{name} y")
    fused = gpu_forward(inp, stagewise=False)
    assert np.array_equal(fused["y"], got["y"]), "fused forward differs from the stage calls"
    print(f"[split] {name}: max rel err {err:.3g}", flush=True)


# gate/up: 286 tiles, 35 or 36 per XCD, so one whole round and a last round
# of 3 or 4 tiles split in 2 parts (30 split, 256 whole); down: every tile
# split in 2
MIXED = syn.CONFIGS["mixtral"].replace(name="mixed_bf16", T=1100, D=2048, F=3328)
GIVE_UP = {"mixed_bf16": MIXED, "split2_mxfp4": SPLIT_CASES["split2_mxfp4"][0],
           "split2_a8": SPLIT_CASES["split2_a8"][0], "split8_down": SPLIT_CASES["split8_down"][0]}


def _lost_rows_cols(cfg, h_or_y, which, A):
    """Boolean [A, N] map of NaN outputs (MXFP8 H: a block with the NaN
    scale 0xFF marks its 32 columns)."""
    if which == "H" and cfg.wdt == syn.MXFP4_A8:
        rows, F = cfg.T * cfg.k, cfg.F
        b = h_or_y.reshape(-1).view(torch.uint8).cpu().numpy()
        G = (F + 511) // 512
        sc = b[rows * F:rows * F + G * rows * 16].reshape(G, rows, 16)
        sc = sc.transpose(1, 0, 2).reshape(rows, G * 16)[:A, :F // 32]
        return np.repeat(sc == 0xFF, 32, axis=1)
    v = h_or_y.float().cpu().numpy()[:A]
    return np.isnan(v)


def _bits(cfg, t, which, A):
    """The bytes of the first A rows (MXFP8 H: their codes and scales)."""
    if which == "H" and cfg.wdt == syn.MXFP4_A8:
        rows, F = cfg.T * cfg.k, cfg.F
        b = t.reshape(-1).view(torch.uint8).cpu().numpy()
        G = (F + 511) // 512
        sc = b[rows * F:rows * F + G * rows * 16].reshape(G, rows, 16)[:, :A]
        return np.concatenate([b[:A * F], sc.reshape(-1)])
    return t.reshape(t.shape[0], -1).view(torch.uint8).cpu().numpy()[:A]


@pytest.mark.parametrize("name", list(GIVE_UP))
def test_split_give_up_stores_nan_in_exactly_the_split_tiles(name):
    """With the flag wait set to 0 polls, the last part of every split tile
    gives up at once: its outputs are NaN, every other output is bit-equal
    to the normal run's, all kernels exit normally, and a normal run after
    it (flags zeroed again) reproduces the first one."""
    cfg = GIVE_UP[name]
    print(f"[split] give-up {name}: {cfg}", flush=True)
    inp = syn.make_inputs(cfg)
    c, x, W_r, bias, w = upload.to_device(inp)
    idx, tw, _ = moe.route(c, x, W_r, bias)
    d = moe.dispatch(c, idx, x)
    torch.cuda.synchronize()
    off = d["offsets"].cpu().numpy()
    A = int(off[-1])
    tiles = {g: [t for t in tp.plan(off, *((cfg.D, cfg.F) if g == "gate_up" else (cfg.F, cfg.D)),
                                    g == "gate_up", wide=_wide(cfg))] for g in ("gate_up", "down")}
    n_split = {g: sum(t.S > 1 for t in ts) for g, ts in tiles.items()}
    assert n_split["gate_up"] + n_split["down"] > 0
    ws = moe.workspace(c, moe.WS_EXPERT_FFN, x.device)
    rows = cfg.T * cfg.k

    def run():
        H = torch.empty((rows, cfg.F), dtype=torch.bfloat16, device=x.device)
        y = torch.empty((rows, cfg.D), dtype=torch.float32, device=x.device)
        moe.expert_gate_up(c, d["x_perm"], d["offsets"], w, H, ws)
        return H, y

    H0, y0 = run()
    moe.expert_down(c, H0, d["offsets"], w, y0, ws)
    torch.cuda.synchronize()
    prev = moe.set_split_wait(0)
    try:
        H1, y1 = run()
        moe.expert_down(c, H0, d["offsets"], w, y1, ws)   # down on the good H
        torch.cuda.synchronize()
    finally:
        moe.set_split_wait(prev)
    H2, y2 = run()
    moe.expert_down(c, H2, d["offsets"], w, y2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(cfg, H2, "H", A), _bits(cfg, H0, "H", A)), \
        "flags left raised by the give-up run"
    assert np.array_equal(_bits(cfg, y2, "y", A), _bits(cfg, y0, "y", A))
    for which, out, good, g, N in (("H", H1, H0, "gate_up", cfg.F), ("y", y1, y0, "down", cfg.D)):
        want = np.zeros((A, N), bool)
        for t in tiles[g]:
            if t.S > 1:
                want[t.row0:min(t.row0 + tp.TM, t.row_end), t.col0:t.col1] = True
        lost = _lost_rows_cols(cfg, out, which, A)
        assert np.array_equal(lost, want), (f"{which}: {int((lost & ~want).sum())} NaN outside "
                                            f"split tiles, {int((want & ~lost).sum())} missing")
        assert not _lost_rows_cols(cfg, good, which, A).any()
        if not (which == "H" and cfg.wdt == syn.MXFP4_A8):
            ob = out.float().cpu().numpy()[:A]
            gb = good.float().cpu().numpy()[:A]
            assert np.array_equal(ob[~want], gb[~want]), f"{which}: whole tiles changed"
    print(f"[split] {name}: split tiles gate/up {n_split['gate_up']} down {n_split['down']}",
          flush=True)
