"""The host replica of the GEMM tile schedule: every output tile exactly
once, split only in an XCD's last partial round, and the small shapes the
split-tile GPU tests use really split."""
import numpy as np

import tile_plan as tp
from split_cases import SPLIT_CASES, split_offsets


def test_every_tile_once_and_rows_covered():
    offsets = np.array([0, 100, 100, 700, 1234, 1300], np.int64)
    for swiglu, N in ((True, 1000), (False, 4096)):
        tiles = tp.plan(offsets, K=4096, N=N, swiglu=swiglu)
        cover = np.zeros((int(offsets[-1]), N), np.int32)
        for t in tiles:
            cover[t.row0:min(t.row0 + tp.TM, t.row_end), t.col0:t.col1] += 1
        assert (cover == 1).all()


def test_split_cases_split():
    for name, (cfg, want) in SPLIT_CASES.items():
        off = split_offsets(cfg)
        for gemm, S in want.items():
            swiglu = gemm == "gate_up"
            K, N = (cfg.D, cfg.F) if swiglu else (cfg.F, cfg.D)
            got = {t.S for t in tp.plan(off, K, N, swiglu)}
            assert S in got, (name, gemm, got)
