"""Host replica of the grouped GEMMs' tile schedule (integer logic only).

It restates, for the tests, how the GEMM kernels map workgroups to output
tiles: the tile map built from the segment offsets (M-tiles of 256 rows, per
expert, in expert order), the expert-major tile order (groups of up to 16 of
an expert's M-tiles, N-tile major inside a group), the cut of the tiles into
8 contiguous ranges (one per XCD) and the split along K of each tile of an
XCD's last, partial round of 32. Tests use it to choose shapes where tiles
really are split and to know which output rows and columns each split tile
owns; it computes no layer arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass

TM = 256          # rows per M-tile
CUS_PER_XCD = 32
MAX_SPLIT = 8
MIN_PART_K = 1024
GROUP_M = 16


@dataclass(frozen=True)
class Tile:
    e: int        # expert
    row0: int     # first segment row
    row_end: int  # end of the expert's segment
    col0: int     # first output column (H column f for gate/up, y_perm column for down)
    col1: int     # one past the last output column (clipped to N)
    S: int        # K-parts of the tile (1: not split)


def m_tiles(offsets):
    """The tile map: (expert, first row) of every M-tile, in expert order."""
    out = []
    for e in range(len(offsets) - 1):
        seg = int(offsets[e + 1]) - int(offsets[e])
        for i in range((seg + TM - 1) // TM):
            out.append((e, int(offsets[e]) + TM * i))
    return out


def _expert_tile(t, MT, NT, tmap, offsets):
    g = t // NT
    e, r0 = tmap[g]
    seg = int(offsets[e])
    first = g - (r0 - seg) // TM
    m = (int(offsets[e + 1]) - seg + TM - 1) // TM
    r = t - first * NT
    gi = r // (GROUP_M * NT)
    gsz = min(GROUP_M, m - gi * GROUP_M)
    rr = r - gi * GROUP_M * NT
    return first + gi * GROUP_M + rr % gsz, rr // gsz


def plan(offsets, K: int, N: int, swiglu: bool, splits: bool = True):
    """Every tile of one grouped GEMM launch with its K-part count."""
    tmap = m_tiles(offsets)
    MT = len(tmap)
    NT = (N + 127) // 128 if swiglu else (N + 255) // 256
    width = 128 if swiglu else 256
    total = MT * NT
    tiles = {}
    for xcd in range(8):
        lo, hi = total * xcd // 8, total * (xcd + 1) // 8
        whole = (hi - lo) // CUS_PER_XCD * CUS_PER_XCD
        rem = hi - lo - whole
        S = 1
        if splits and rem > 0:
            S = max(1, min(MAX_SPLIT, CUS_PER_XCD // rem, K // MIN_PART_K))
        for t in range(lo, hi):
            s = S if t >= lo + whole else 1
            mt, nt = _expert_tile(t, MT, NT, tmap, offsets)
            e, r0 = tmap[mt]
            assert (mt, nt) not in tiles
            tiles[(mt, nt)] = Tile(e, r0, int(offsets[e + 1]), nt * width,
                                   min(N, (nt + 1) * width), s)
    assert len(tiles) == total
    return list(tiles.values())


def split_tiles(offsets, K, N, swiglu):
    return [t for t in plan(offsets, K, N, swiglu) if t.S > 1]
