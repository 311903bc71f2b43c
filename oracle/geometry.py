"""Tile geometry of a (T, Y, X) latent token grid cut into 4x4x4 tiles.

Follows:
  * "video_sparse_attn" page, construct_variable_block_sizes: tile counts
    per axis, per-axis tile extents where the last tile holds the remainder,
    and the per-tile valid-token count as the product of the three extents,
    flattened with the time tile outermost and the width tile innermost.
  * "bsa_attn" page, get_tile_partition_indices: raster token ids
    arange(T*H*W) reshaped to (T, H, W); tiles visited t-tile, then h-tile,
    then w-tile; each tile contributes its clipped sub-block flattened in
    row-major order.
  * "video_sparse_attn_h3" page, tile(): tiles live in a zero-padded buffer
    of tile_elems slots each.

Reading taken where the pages leave it open: inside a partial tile the valid
tokens fill slots 0..n_j-1 in the clipped sub-block's row-major order and the
remaining slots are padding (compact, valid first).  Grid axes are written
(T, Y, X) here; the pages call them (T, H, W).
"""
from __future__ import annotations

import math

import numpy as np

TILE = (4, 4, 4)
TILE_ELEMS = TILE[0] * TILE[1] * TILE[2]


def tile_counts(T: int, Y: int, X: int, tile=TILE):
    """Number of tiles along each axis (ceil division)."""
    return (math.ceil(T / tile[0]), math.ceil(Y / tile[1]), math.ceil(X / tile[2]))


def num_tiles(T: int, Y: int, X: int, tile=TILE) -> int:
    nt, ny, nx = tile_counts(T, Y, X, tile)
    return nt * ny * nx


def padded_len(T: int, Y: int, X: int, tile=TILE) -> int:
    return num_tiles(T, Y, X, tile) * tile[0] * tile[1] * tile[2]


def _axis_sizes(dim_len: int, tile: int, n_tiles: int) -> np.ndarray:
    """Extent of each tile along one axis; the last tile keeps the remainder."""
    sizes = np.full(n_tiles, tile, dtype=np.int64)
    remainder = dim_len - (n_tiles - 1) * tile
    sizes[-1] = remainder if remainder > 0 else tile
    return sizes


def occupancy(T: int, Y: int, X: int, tile=TILE) -> np.ndarray:
    """Valid tokens per tile, int64 [Nt], tiles in (t, y, x) order."""
    nt, ny, nx = tile_counts(T, Y, X, tile)
    st = _axis_sizes(T, tile[0], nt)
    sy = _axis_sizes(Y, tile[1], ny)
    sx = _axis_sizes(X, tile[2], nx)
    return (st[:, None, None] * sy[None, :, None] * sx[None, None, :]).reshape(-1)


def tile_partition_indices(T: int, Y: int, X: int, tile=TILE) -> np.ndarray:
    """Raster token ids listed in tile-contiguous (unpadded) order."""
    ts, ys, xs = tile
    ids = np.arange(T * Y * X, dtype=np.int64).reshape(T, Y, X)
    parts = []
    for a in range(math.ceil(T / ts)):
        for b in range(math.ceil(Y / ys)):
            for c in range(math.ceil(X / xs)):
                parts.append(ids[a * ts:min(a * ts + ts, T),
                                 b * ys:min(b * ys + ys, Y),
                                 c * xs:min(c * xs + xs, X)].reshape(-1))
    return np.concatenate(parts)


def reverse_tile_partition_indices(T: int, Y: int, X: int, tile=TILE) -> np.ndarray:
    """Inverse of tile_partition_indices (argsort of it)."""
    return np.argsort(tile_partition_indices(T, Y, X, tile), kind="stable")


def token_slots(T: int, Y: int, X: int, tile=TILE) -> np.ndarray:
    """For each raster token, its slot in the zero-padded tile buffer.

    Tile j owns slots [j*E, (j+1)*E) with E = prod(tile); its valid tokens take
    the first n_j slots in the order the partition lists them.
    """
    E = tile[0] * tile[1] * tile[2]
    perm = tile_partition_indices(T, Y, X, tile)
    occ = occupancy(T, Y, X, tile)
    slots = np.empty(T * Y * X, dtype=np.int64)
    pos = 0
    for j, n in enumerate(occ):
        slots[perm[pos:pos + n]] = j * E + np.arange(n)
        pos += n
    assert pos == T * Y * X
    return slots


def tile_coords(T: int, Y: int, X: int, tile=TILE) -> np.ndarray:
    """(a, b, c) tile coordinates of every tile id j, int64 [Nt, 3]."""
    nt, ny, nx = tile_counts(T, Y, X, tile)
    a, b, c = np.meshgrid(np.arange(nt), np.arange(ny), np.arange(nx), indexing="ij")
    return np.stack([a.reshape(-1), b.reshape(-1), c.reshape(-1)], axis=1)
