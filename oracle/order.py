"""Oracle of the visit orders (test infrastructure only): for pixel-centre
queries, and for queries given by a point each.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module; the HIP library never calls it and the two share no code.

The queries are the centres of the pyramid's pixels in flattened order (query
s is pixel s), the encoder case where each query's reference point is its own
position on the feature map ("What is Deformable Attention", reference
position; "3D Attention That Knows Where to Look", recipe step 1).  The order
the library builds is defined as a sort: every pixel gets the cell of a grid
of 2^10 cells per axis over the unit square (cube) that holds its normalized
centre, floor((2j+1) * 2^10 / (2E)) along an axis of extent E; the cell's
Z-order (Morton) key interleaves the cell coordinates bit by bit, x lowest;
and the pixels are sorted by (key, level, index in the level), or by (level,
key, index) for the level-major order.  This module computes exactly that
with integer arithmetic and one stable sort (the library instead counts each
pixel's rank in closed form, without sorting).

Queries whose reference points depend on the data (the decoder's learned
reference points, "What is Deformable Attention", reference position) are
ordered by one point each, in normalized coordinates: along every axis the
point gets the cell floor(x * 2^B) of a grid of 2^B cells over the unit
interval, clamped to [0, 2^B - 1] (a NaN coordinate counts as 0), with B = 16
in 2D and 10 in 3D (a 32- or 30-bit key); the product x * 2^B is taken in
fp32, where scaling by a power of two is exact.  The queries are sorted by
(Morton key of the cells, query index).
"""
from __future__ import annotations

import numpy as np

CELL_BITS = 10


def pixel_cells(shapes, dims: int):
    """Per pixel of the flattened pyramid: (level, index in level, cell
    coordinates [S, dims] with column 0 = x)."""
    levels, index, cells = [], [], []
    for l, shp in enumerate(shapes):
        ext = [int(e) for e in shp]            # (H, W) or (Z, H, W)
        n = int(np.prod(ext))
        r = np.arange(n, dtype=np.int64)
        # raster index -> coordinates, x (along W) fastest
        coords = []
        rest = r
        for e in reversed(ext):                # W, then H, then Z
            coords.append(rest % e)
            rest = rest // e
        c = np.stack([((2 * j + 1) << CELL_BITS) // (2 * e)
                      for j, e in zip(coords, reversed(ext))], axis=1)
        levels.append(np.full(n, l, dtype=np.int64))
        index.append(r)
        cells.append(c)
    return np.concatenate(levels), np.concatenate(index), np.concatenate(cells)


def morton_key(cells: np.ndarray, bits: int = CELL_BITS) -> np.ndarray:
    """Z-order key of cell coordinates [S, dims]: bit b of axis d goes to key
    bit dims*b + d."""
    dims = cells.shape[1]
    key = np.zeros(cells.shape[0], dtype=np.int64)
    for b in range(bits):
        for d in range(dims):
            key |= ((cells[:, d] >> b) & 1) << (dims * b + d)
    return key


def point_bits(dims: int) -> int:
    """Cells per axis (as a power of two) of the points order."""
    return 16 if dims == 2 else 10


def point_cells(points) -> np.ndarray:
    """Cell coordinates [Lq, dims] of points [Lq, dims] (column 0 = x)."""
    pts = np.asarray(points, dtype=np.float32)
    bits = point_bits(pts.shape[1])
    scaled = pts * np.float32(1 << bits)            # exact: a power of two
    scaled = np.where(np.isnan(scaled), np.float32(0), scaled)
    return np.clip(np.floor(scaled), 0, (1 << bits) - 1).astype(np.int64)


def points_order_oracle(points) -> np.ndarray:
    """The visit order (int64 [Lq]) of queries given by one point each: entry
    r is the query of rank r by (Morton key of its cell, query index)."""
    cells = point_cells(points)
    key = morton_key(cells, point_bits(cells.shape[1]))
    return np.lexsort((np.arange(len(key)), key)).astype(np.int64)


def query_order_oracle(shapes, level_major: bool) -> np.ndarray:
    """The visit order (int64 [S]): entry r is the pixel of rank r."""
    shapes = [tuple(int(e) for e in s) for s in shapes]
    dims = len(shapes[0])
    level, index, cells = pixel_cells(shapes, dims)
    key = morton_key(cells)
    # np.lexsort sorts by the last key first
    if level_major:
        order = np.lexsort((index, key, level))
    else:
        order = np.lexsort((index, level, key))
    return order.astype(np.int64)
