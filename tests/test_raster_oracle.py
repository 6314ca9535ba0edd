"""Pins of the oracle's block-id -> tile maps (pure integer work, CPU only)."""
import pytest

from conftest import read_golden
from oracle import raster


def test_fig19_tile_space_indexing():
    g = read_golden("tile_space_fig19.txt")
    shape, tile = g["array_shape"][0], g["tile_shape"][0]
    assert list(raster.tile_grid(shape, tile)) == g["tile_grid"][0]
    (r0, r1), (c0, c1) = raster.tile_elements(shape, tile, g["tile_index"][0])
    assert [r0, c0] == g["first_element"][0]
    assert [r1 - 1, c1 - 1] == g["last_element"][0]


def test_cdiv_example():
    assert raster.cdiv(7, 4) == 2 and raster.cdiv(8, 4) == 2 and raster.cdiv(0, 4) == 0


def _unique_block_loads(tiles, k_blocks):
    a = {(m, k) for (m, _) in tiles for k in range(k_blocks)}
    b = {(k, n) for (_, n) in tiles for k in range(k_blocks)}
    return len(a) + len(b)


def test_fig2_grouped_order_loads_fewer_blocks():
    g = read_golden("swizzle_2x2_fig2.txt")
    gm, gn = g["grid"][0]
    kb = g["k_blocks"][0][0]
    n_out = g["outputs"][0][0]
    G = g["group_size_m"][0][0]
    linear = [raster.linear_2d(gn, 1, b) for b in range(n_out)]
    grouped = [raster.swizzle_2d_from_bid(gm, gn, 1, 1, G, b) for b in range(n_out)]
    assert sorted(grouped) == [(0, 0), (0, 1), (1, 0), (1, 1)]
    assert _unique_block_loads(linear, kb) == g["linear_loads"][0][0]
    assert _unique_block_loads(grouped, kb) == g["grouped_loads"][0][0]


@pytest.mark.parametrize("G", [1, 2, 3, 8])
def test_both_page_swizzles_are_bijections(G):
    for gm in range(1, 20):
        for gn in range(1, 20):
            n = gm * gn
            p1 = [raster.swizzle_2d_from_bid(gm, gn, 1, 1, G, b) for b in range(n)]
            p2 = [raster.swizzle_2d_p2(gm, gn, 1, 1, G, b) for b in range(n)]
            want = {(i, j) for i in range(gm) for j in range(gn)}
            assert set(p1) == want and len(p1) == n
            assert set(p2) == want and len(p2) == n
            # identical on every full group
            full = (gm // G) * G * gn
            assert p1[:full] == p2[:full]


@pytest.mark.parametrize("X", [1, 2, 8])
def test_xcd_remap_bijection_and_contiguity(X):
    for W in list(range(1, 70)) + [240, 256, 1024, 1536]:
        ids = [raster.xcd_remap(w, W, X) for w in range(W)]
        assert sorted(ids) == list(range(W))
        for x in range(X):
            mine = [ids[w] for w in range(x, W, X)]
            assert mine == list(range(mine[0], mine[0] + len(mine))) if mine else True
