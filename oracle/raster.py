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
  the group is taken from the id modulo (actual group size * grid_n) before
  the modulo by the group size. The two forms agree on full groups and may
  order the last, partial group differently.
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


def cdiv(a: int, b: int) -> int:
    """Ceiling division (page 2, section 5.6: cdiv(7, 4) = 2)."""
    return -(-a // b)


def swizzle_2d_from_bid(M: int, N: int, tm: int, tn: int, group_size_m: int, bid: int):
    """Page 1, section "Swizzle": block id -> (tile row, tile column)."""
    num_bid_m = cdiv(M, tm)
    num_bid_n = cdiv(N, tn)
    num_bid_in_group = group_size_m * num_bid_n
    group_id = bid // num_bid_in_group
    first_bid_m = group_id * group_size_m
    group_size = min(num_bid_m - first_bid_m, group_size_m)
    bid_m = first_bid_m + (bid % group_size)
    bid_n = (bid % num_bid_in_group) // group_size
    return bid_m, bid_n


def swizzle_2d_p2(M: int, N: int, tm: int, tn: int, group_size: int, linear_id: int):
    """Page 2, section 7.1: block id -> (tile row, tile column)."""
    grid_m = cdiv(M, tm)
    grid_n = cdiv(N, tn)
    group_id = linear_id // (group_size * grid_n)
    first_row_in_group = group_id * group_size
    group_size_actual = min(grid_m - first_row_in_group, group_size)
    within_group = linear_id % (group_size_actual * grid_n)
    bidx = first_row_in_group + (within_group % group_size_actual)
    bidy = within_group // group_size_actual
    return bidx, bidy


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
