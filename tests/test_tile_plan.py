"""The host replica of the GEMM tile schedule: every output tile exactly
once, split only in an XCD's last partial round, and the small shapes the
split-tile GPU tests use really split."""
import numpy as np

import tile_plan as tp
from split_cases import SPLIT_CASES, split_offsets
from mixture_experts_layer_25_amd import synthetic as syn


def test_every_tile_once_and_rows_covered():
    # segments of 100, 0, 600 (2 full M-tiles + 88), 534 (2 + 22), 66 and 400
    # (1 + 144) rows: wide tails, an empty expert and a regular tail
    offsets = np.array([0, 100, 100, 700, 1234, 1300, 1700], np.int64)
    for wide in (True, False):
        for swiglu, N in ((True, 1000), (False, 4096)):
            tiles = tp.plan(offsets, K=4096, N=N, swiglu=swiglu, wide=wide)
            cover = np.zeros((int(offsets[-1]), N), np.int32)
            for t in tiles:
                rows = tp.TM_WIDE if t.wide else tp.TM
                assert t.wide <= wide and (not t.wide or t.row_end - t.row0 <= rows)
                cover[t.row0:min(t.row0 + rows, t.row_end), t.col0:t.col1] += 1
            assert (cover == 1).all()
            n_wide = sum(t.wide for t in tiles)
            assert n_wide == (4 * -(-N // (256 if swiglu else 512)) if wide else 0)


def test_split_cases_split():
    for name, (cfg, want) in SPLIT_CASES.items():
        off = split_offsets(cfg)
        for gemm, S in want.items():
            swiglu = gemm == "gate_up"
            K, N = (cfg.D, cfg.F) if swiglu else (cfg.F, cfg.D)
            got = {t.S for t in tp.plan(off, K, N, swiglu, wide=syn.is_mx(cfg.wdt))}
            assert S in got, (name, gemm, got)
