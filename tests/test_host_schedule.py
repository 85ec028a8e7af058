"""Host mirror of the persistent forward products' tile list and walk (bench.tile_schedule), checked on
the CPU against counts worked out by hand: the tile height of a dense (one-expert) product, band tiles,
empty experts, the balancing walk for a partial last round, and that every tile is dealt exactly once."""
import numpy as np
import pytest

import bench


def test_dense_product_takes_256_row_tiles_when_they_fill_the_grid():
    # 4096 rows, 16 column tiles: 13 x 16 = 208 tiles of up to 320 rows leave 48 of 256 CUs idle;
    # 16 x 16 = 256 tiles of 256 rows are one whole round on every XCD
    s = bench.tile_schedule([4096], 4096)
    assert (s["tiles"], s["tile_rows_max"], s["workgroup_tiles_max"]) == (256, 256, 1)
    # 28 column tiles: 364 or 448 tiles, two rounds either way -> 256-row tiles
    s = bench.tile_schedule([4096], 7168)
    assert (s["tiles"], s["tile_rows_max"]) == (448, 256)
    # 2500 rows: one partial round either way -> the fewest tiles (320-row band tiles)
    for cols, tiles in ((4096, 8 * 16), (7168, 8 * 28)):
        s = bench.tile_schedule([2500], cols)
        assert (s["tiles"], s["tile_rows_max"]) == (tiles, 320)


def test_several_experts_keep_band_tiles():
    # two experts of 2048 rows: 14 row tiles at 320, 16 at 256 (whole rounds) -> still 320 (several experts)
    s = bench.tile_schedule([2048, 0, 2048], 4096)
    assert (s["tiles"], s["tile_rows_max"]) == (14 * 16, 320)
    assert s["empty_experts"] == 1 and s["tiles_of_empty_experts"] == 0
    # 300 rows: one band tile (257-320 rows), 321 rows: two tiles
    assert bench.tile_schedule([300, 321, 0, 1], 256)["tiles_per_expert"] == [1, 2, 0, 1]


def test_whole_rounds_and_balance():
    # 128 experts of 256 rows, 6 column tiles: 768 tiles, 96 per XCD, 3 per workgroup, contiguous split
    s = bench.tile_schedule([256] * 128, 1536)
    assert s["tiles"] == 768 and s["tiles_per_xcd"] == [96] * 8 and s["workgroup_tiles_max"] == 3
    assert not s["balanced_walk"]
    # a partial last round with few rounds balances: tallest first, row tile R to XCD R mod 8
    counts = [2714, 1171, 719, 473, 384, 320, 246, 219] + [100] * 22 + [0, 0]
    s = bench.tile_schedule(counts, 1536)
    assert s["balanced_walk"] and s["tiles"] == sum(s["tiles_per_xcd"])
    assert s["tiles_of_empty_experts"] == 0


@pytest.mark.parametrize("seed", range(6))
def test_every_tile_dealt_once(seed):
    g = np.random.default_rng(seed)
    E = int(g.integers(1, 300))
    counts = [int(c) for c in g.integers(0, 900, size=E)]
    for cols in (136, 1536, 4096):
        s = bench.tile_schedule(counts, cols)
        ntn = (cols + 255) // 256
        assert s["tiles"] == sum(s["tiles_per_expert"]) == sum(s["tiles_per_xcd"])
        assert all(t % ntn == 0 for t in s["tiles_per_expert"])
        assert all(t == 0 for t, c in zip(s["tiles_per_expert"], counts) if c == 0)
        rows_max = s["tile_rows_max"]
        assert all(t // ntn == (c + rows_max - 1) // rows_max for t, c in zip(s["tiles_per_expert"], counts) if c)
