"""Block-id -> output-tile maps, written from the pages (TEST INFRASTRUCTURE ONLY).

Pure integer Python, used to check the product library's own rasterization.
Which tile a block computes never changes C (tiles are independent), so these
maps are checked for what is unique: the pages' formula where the library
claims to follow it, and the bijection property everywhere.

* ``swizzle_2d_from_bid``: page 1 ("Using NVIDIA CUDA Tile to write a
  high-performance matrix multiply"), section "Performance optimization:
  Swizzle". Blocks are grouped GROUP_SIZE_M tile-rows at a time; inside a
  group, consecutive block ids walk down the group's rows first, then move to
  the next tile-column. The page uses GROUP_SIZE_M = 8.
* ``swizzle_2d_p2``: page 2 ("CUDA 13.1 new feature: the Tile programming
  model"), section 7.1 "2D Block Swizzle". The same grouping; the row inside
  the group follows the id's offset within its group rather than the id
  itself. The two forms agree on full groups and may order the last,
  partial group differently.
  Both are written here as an enumeration of the order the pages describe
  (bands of tile-rows, each served column by column), not as the pages'
  per-id formulas; the tests check the product's per-id map against it.
* ``tile_elements``: page 4 (CUDA programming guide 13.4.2, chapter "Writing
  tile kernels"), section 2.4.6.1 and its Figure 19: a partition view splits
  an array into non-overlapping tiles of a fixed shape; tile index (i, j)
  covers elements [i*th, i*th + th) x [j*tw, j*tw + tw), clipped to the array.
* ``xcd_remap``: not on the pages (they do not discuss chiplets). Its
  definition: with W blocks dispatched round-robin over X dies (block w goes
  to die w mod X), renumber the blocks so that each die receives one
  contiguous range of logical ids, die x taking ids in increasing order of w.
"""
from __future__ import annotations

from functools import lru_cache


def cdiv(a: int, b: int) -> int:
    """Ceiling division (page 2, section 5.6: cdiv(7, 4) = 2)."""
    return -(-a // b)


@lru_cache(maxsize=None)
def _grouped_order(rows: int, cols: int, height: int, rotate_by_global_id: bool):
    """Every tile (row, column) of a rows x cols tile grid, in the order the
    grouped raster hands them to block ids 0, 1, 2, ...

    Tile-rows are cut into bands of `height` consecutive rows (the last band
    keeps what is left). Bands are served top to bottom. Inside a band of h
    rows, each tile-column in turn, left to right, receives h consecutive ids,
    one per row of the band, so ids run down a column before moving right.
    The row an id lands on inside its column is its offset in the band modulo
    h (page 2's wording), or, with rotate_by_global_id, the block id itself
    modulo h (page 1's wording); on full bands both are the same, because a
    full band starts at a multiple of h."""
    order = []
    for top in range(0, rows, height):
        h = min(height, rows - top)
        band_start = len(order)
        for offset in range(h * cols):
            col = offset // h
            r = (band_start + offset if rotate_by_global_id else offset) % h
            order.append((top + r, col))
    return tuple(order)


def swizzle_2d_from_bid(M: int, N: int, tm: int, tn: int, group_size_m: int, bid: int):
    """Page 1, section "Swizzle": block id -> (tile row, tile column) for an
    M x N output cut into tm x tn tiles, bands of group_size_m tile-rows."""
    return _grouped_order(cdiv(M, tm), cdiv(N, tn), group_size_m, True)[bid]


def swizzle_2d_p2(M: int, N: int, tm: int, tn: int, group_size: int, linear_id: int):
    """Page 2, section 7.1: block id -> (tile row, tile column); the row inside
    the last, partial band follows the id's offset within that band."""
    return _grouped_order(cdiv(M, tm), cdiv(N, tn), group_size, False)[linear_id]


def linear_2d(N: int, tn: int, bid: int):
    """Row-major (unswizzled) order: consecutive ids walk along a tile-row."""
    grid_n = cdiv(N, tn)
    return bid // grid_n, bid % grid_n


def tile_elements(shape, tile_shape, index):
    """Page 4, Figure 19: element ranges [start, stop) per axis of a tile."""
    out = []
    for extent, t, i in zip(shape, tile_shape, index):
        start = i * t
        out.append((start, min(start + t, extent)))
    return tuple(out)


def tile_grid(shape, tile_shape):
    """Page 4, Figure 19: number of tiles per axis of a partition view."""
    return tuple(cdiv(e, t) for e, t in zip(shape, tile_shape))


def xcd_remap(w: int, W: int, X: int) -> int:
    """Logical id of block w when W blocks go round-robin to X dies and each
    die is to receive one contiguous range of logical ids."""
    x = w % X
    # blocks of die x, in dispatch order: x, x + X, x + 2X, ...
    before = sum(len(range(d, W, X)) for d in range(x))
    return before + w // X
