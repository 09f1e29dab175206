"""Host replica of the grouped GEMMs' tile schedule (integer logic only).

It restates, for the tests, how the GEMM kernels map workgroups to output
tiles: the tile map built from the segment offsets (M-tiles of 256 rows, per
expert, in expert order; with wide tiles on, an expert's last M-tile of at
most 128 rows is listed separately, after all regular ones, as a wide tile
of twice the columns), the expert-major order of the regular tiles (groups
of up to 16 of an expert's M-tiles, N-tile major inside a group) followed by
the wide tiles (M-tile major), the cut of each of the two lists into 8
contiguous ranges (one per XCD, which runs its regular range, then its wide
range) and the split along K of each tile of an XCD's last, partial round of
32. Tests use it to choose shapes where tiles really are split and
to know which output rows and columns each split tile owns; it computes no
layer arithmetic. Wide tiles are on for MXFP4 weights and off for bf16
weights.
"""
from __future__ import annotations

from dataclasses import dataclass

TM = 256          # rows per M-tile
TM_WIDE = 128     # a last M-tile of at most this many rows is wide
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
    wide: bool = False


def _regular_count(rows, wide):
    full, rem = divmod(rows, TM)
    return full + (1 if rem > (TM_WIDE if wide else 0) else 0)


def m_tiles(offsets, wide=True):
    """The tile map: (expert, first row) of every regular M-tile, in expert
    order, then of every wide M-tile."""
    reg, wid = [], []
    for e in range(len(offsets) - 1):
        seg = int(offsets[e + 1]) - int(offsets[e])
        nreg = _regular_count(seg, wide)
        for i in range(nreg):
            reg.append((e, int(offsets[e]) + TM * i))
        if wide and seg % TM and seg % TM <= TM_WIDE:
            wid.append((e, int(offsets[e]) + TM * (seg // TM)))
    return reg, wid


def _expert_tile(t, MT, NT, tmap, offsets, wide):
    g = t // NT
    e, r0 = tmap[g]
    seg = int(offsets[e])
    first = g - (r0 - seg) // TM
    m = _regular_count(int(offsets[e + 1]) - seg, wide)
    r = t - first * NT
    gi = r // (GROUP_M * NT)
    gsz = min(GROUP_M, m - gi * GROUP_M)
    rr = r - gi * GROUP_M * NT
    return first + gi * GROUP_M + rr % gsz, rr // gsz


def plan(offsets, K: int, N: int, swiglu: bool, splits: bool = True, wide: bool = True):
    """Every tile of one grouped GEMM launch with its K-part count."""
    reg, wid = m_tiles(offsets, wide)
    MT, MW = len(reg), len(wid)
    NT = (N + 127) // 128 if swiglu else (N + 255) // 256
    NTW = (N + 255) // 256 if swiglu else (N + 511) // 512
    width = 128 if swiglu else 256
    R, W = MT * NT, MW * NTW
    tiles = {}
    for xcd in range(8):
        r_lo, r_hi = R * xcd // 8, R * (xcd + 1) // 8
        w_lo, w_hi = W * xcd // 8, W * (xcd + 1) // 8
        # this XCD's list: its range of regular tiles, then its wide range
        lst = [("r", t) for t in range(r_lo, r_hi)] + [("w", u) for u in range(w_lo, w_hi)]
        whole = len(lst) // CUS_PER_XCD * CUS_PER_XCD
        rem = len(lst) - whole
        S = 1
        if splits and rem > 0:
            S = max(1, min(MAX_SPLIT, CUS_PER_XCD // rem, K // MIN_PART_K))
        for li, (kind, t) in enumerate(lst):
            s = S if li >= whole else 1
            if kind == "r":
                mt, nt = _expert_tile(t, MT, NT, reg, offsets, wide)
                e, r0 = reg[mt]
                w = width
                key = ("r", mt, nt)
            else:
                mt, nt = divmod(t, NTW)
                e, r0 = wid[mt]
                w = 2 * width
                key = ("w", mt, nt)
            assert key not in tiles
            tiles[key] = Tile(e, r0, int(offsets[e + 1]), nt * w, min(N, (nt + 1) * w), s,
                              key[0] == "w")
    assert len(tiles) == R + W
    return list(tiles.values())


def split_tiles(offsets, K, N, swiglu, wide=True):
    return [t for t in plan(offsets, K, N, swiglu, wide=wide) if t.S > 1]
