"""CPU model of the workgroup -> output-tile mapping of the pipelined kernel (no GPU).

The model restates `tile_of` in csrc/gemm_kernels.hpp.  Workgroups are dispatched
round-robin over the 8 XCDs (workgroup w runs on XCD w % 8); with the remap on, XCD x
is handed one contiguous range of the raster order, the x-th of 8 near-equal ranges.
The raster order walks groups of `group_m` tile rows, column by column inside a group,
so that the workgroups resident at one time on one XCD share few A row panels and B
column panels (the L2 of an XCD is its own).

Checked here for many grids: the mapping is a bijection onto the tiles (no tile lost or
computed twice, also for a last group of fewer rows and tile counts that 8 does not
divide), each XCD's tiles are one contiguous range of the raster order, and the panel
counts behind the measured L2 hit rate: at 8192^3 with 256x256 tiles every XCD's 32
resident tiles form a 4 x 8 block (12 panels for 64 panel reads, an ideal hit rate of
81.25% when the tiles advance through K together; the counters read 80.3%), while the
same grid without the remap gives each XCD every 8th tile of the raster: 2 rows and 16
columns, 18 panels.
"""

import pytest


def tile_of(wg, tiles_m, tiles_n, group_m, xcd_remap):
    T = tiles_m * tiles_n
    if xcd_remap:
        x, i, q, r = wg & 7, wg >> 3, T >> 3, T & 7
        wg = x * q + min(x, r) + i
    gsz = group_m * tiles_n
    g = wg // gsz
    first = g * group_m
    gm = min(tiles_m - first, group_m)
    inner = wg - g * gsz
    return first + inner % gm, inner // gm


GRIDS = [(1, 1), (1, 7), (3, 1), (5, 9), (7, 8), (12, 20), (16, 16), (17, 17), (32, 32),
         (33, 5), (4, 64), (64, 4)]


@pytest.mark.parametrize("tiles_m,tiles_n", GRIDS)
@pytest.mark.parametrize("group_m", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("xcd_remap", [0, 1])
def test_mapping_is_a_bijection(tiles_m, tiles_n, group_m, xcd_remap):
    T = tiles_m * tiles_n
    seen = {tile_of(w, tiles_m, tiles_n, group_m, xcd_remap) for w in range(T)}
    assert len(seen) == T
    assert all(0 <= tm < tiles_m and 0 <= tn < tiles_n for tm, tn in seen)


def _raster_index(tm, tn, tiles_m, tiles_n, group_m):
    # position of a tile in the raster order (the inverse of the mapping without remap)
    g = tm // group_m
    gm = min(tiles_m - g * group_m, group_m)
    return g * group_m * tiles_n + tn * gm + (tm - g * group_m)


@pytest.mark.parametrize("tiles_m,tiles_n", GRIDS)
def test_each_xcd_gets_one_contiguous_range(tiles_m, tiles_n):
    T = tiles_m * tiles_n
    ranges = []
    for x in range(8):
        idx = sorted(_raster_index(*tile_of(w, tiles_m, tiles_n, 4, 1), tiles_m, tiles_n, 4)
                     for w in range(x, T, 8))
        if idx:
            assert idx == list(range(idx[0], idx[0] + len(idx)))
            ranges.append((idx[0], len(idx)))
    # the ranges follow each other in XCD order and differ in length by at most one
    pos = 0
    for start, n in ranges:
        assert start == pos
        pos += n
    assert pos == T
    assert max(n for _, n in ranges) - min(n for _, n in ranges) <= 1


def _resident_panels(tiles_m, tiles_n, group_m, xcd_remap, cus=256):
    """Per XCD, the tile rows and columns of the first `cus` workgroups (one round)."""
    rows = [set() for _ in range(8)]
    cols = [set() for _ in range(8)]
    for w in range(min(cus, tiles_m * tiles_n)):
        tm, tn = tile_of(w, tiles_m, tiles_n, group_m, xcd_remap)
        rows[w % 8].add(tm)
        cols[w % 8].add(tn)
    return rows, cols


def test_8192_cubed_round_is_a_4x8_block_per_xcd():
    # 32 x 32 tiles of 256 x 256; 256 CUs take one round of 256 workgroups, 32 per XCD
    rows, cols = _resident_panels(32, 32, 4, 1)
    for x in range(8):
        assert len(rows[x]) == 4 and len(cols[x]) == 8
        assert max(rows[x]) - min(rows[x]) == 3 and max(cols[x]) - min(cols[x]) == 7
    panels = len(rows[0]) + len(cols[0])
    reads = 2 * 32
    assert 1 - panels / reads == pytest.approx(0.8125)


def test_without_the_remap_an_xcd_spreads_over_many_panels():
    # round-robin dispatch of the plain raster order: XCD x gets every 8th tile
    rows, cols = _resident_panels(32, 32, 4, 0)
    for x in range(8):
        assert (len(rows[x]), len(cols[x])) == (2, 16)


def test_one_round_grids_keep_xcd_blocks_compact():
    # 3072 x 4096 with 192 x 256 tiles (16 x 16): 32 tiles per XCD, a 4 x 8 block each
    rows, cols = _resident_panels(16, 16, 4, 1)
    assert all((len(rows[x]), len(cols[x])) == (4, 8) for x in range(8))
    # 3000 x 5000 with 256 x 256 tiles (12 x 20): 30 tiles per XCD; groups of 4 rows
    # hold 80 tiles, so the ranges of XCDs 2 and 5 straddle a group boundary and touch
    # two groups (8 rows, 8 columns); the others stay in one group (4 rows, 8 columns)
    rows, cols = _resident_panels(12, 20, 4, 1)
    shapes = [(len(rows[x]), len(cols[x])) for x in range(8)]
    assert shapes == [(4, 8), (4, 8), (8, 8), (4, 8), (4, 8), (8, 8), (4, 8), (4, 8)]
    assert all(len({tm // 4 for tm in rows[x]}) <= 2 for x in range(8))
