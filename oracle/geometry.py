"""Tile geometry of a (T, Y, X) latent token grid cut into tiles (4x4x4 by default).

Written from what the pages say the geometry is, not from their listings:
  * "bsa_attn" page (tile partition indices; pre/post-processing): tokens of
    a (T, H, W) grid are numbered in row-major order, raster id
    (t*Y + y)*X + x; the grid is cut into tiles, tiles are visited time tile
    first and width tile last, and each tile lists its own tokens, clipped
    at the grid's edge, in row-major order.
  * "video_sparse_attn" section of the backends page (variable block sizes):
    ceil(dim / tile) tiles per axis, the last one on an axis holding the
    remainder; a tile's block size is its number of valid tokens.
  * "video_sparse_attn_h3" page, tile(): tiles live in a zero-padded buffer
    of tile_elems slots each.

So token (t, y, x) belongs to tile (t // 4, y // 4, x // 4), numbered
j = (a*nY + b)*nX + c, and the tile-contiguous order is a stable sort of the
raster ids by tile id (inside a tile raster order is the sub-block's
row-major order).  Occupancy is a count of tokens per tile id.

Reading taken where the pages leave it open: inside a partial tile the valid
tokens fill slots 0..n_j-1 in that order and the remaining slots are padding
(compact, valid first).  Grid axes are written (T, Y, X) here; the pages
call them (T, H, W).
"""
from __future__ import annotations

import math

import numpy as np

TILE = (4, 4, 4)
TILE_ELEMS = TILE[0] * TILE[1] * TILE[2]
# Tile shapes by token count.  The "video_sparse_attn_h3" page keys its tile
# registry by 64 and 128 tokens without printing the shapes; reading: the
# 64-token tile is 4x4x4 (the configurations') and the 128-token tile doubles
# the innermost (width) axis, 4x4x8.
TILE_SHAPES = {64: (4, 4, 4), 128: (4, 4, 8)}


def tile_elems(tile=TILE) -> int:
    return tile[0] * tile[1] * tile[2]


def tile_counts(T: int, Y: int, X: int, tile=TILE):
    """Number of tiles along each axis (ceil division)."""
    return (math.ceil(T / tile[0]), math.ceil(Y / tile[1]), math.ceil(X / tile[2]))


def num_tiles(T: int, Y: int, X: int, tile=TILE) -> int:
    nt, ny, nx = tile_counts(T, Y, X, tile)
    return nt * ny * nx


def padded_len(T: int, Y: int, X: int, tile=TILE) -> int:
    return num_tiles(T, Y, X, tile) * tile[0] * tile[1] * tile[2]


def token_tile_ids(T: int, Y: int, X: int, tile=TILE) -> np.ndarray:
    """Tile id of every raster token, from its grid coordinates: int64 [L]."""
    _, ny, nx = tile_counts(T, Y, X, tile)
    t, y, x = np.meshgrid(np.arange(T), np.arange(Y), np.arange(X), indexing="ij")
    j = ((t // tile[0]) * ny + y // tile[1]) * nx + x // tile[2]
    return j.reshape(-1).astype(np.int64)


def occupancy(T: int, Y: int, X: int, tile=TILE) -> np.ndarray:
    """Valid tokens per tile (a count of the tokens carrying each tile id), int64 [Nt]."""
    return np.bincount(token_tile_ids(T, Y, X, tile),
                       minlength=num_tiles(T, Y, X, tile)).astype(np.int64)


def tile_order(T: int, Y: int, X: int, tile=TILE) -> np.ndarray:
    """Raster token ids in tile-contiguous (unpadded) order.

    A stable sort of the raster ids by tile id: tiles in increasing j, and
    inside a tile its tokens in increasing raster id.
    """
    return np.argsort(token_tile_ids(T, Y, X, tile), kind="stable")


def token_slots(T: int, Y: int, X: int, tile=TILE) -> np.ndarray:
    """For each raster token, its slot in the zero-padded tile buffer.

    Tile j owns slots [j*E, (j+1)*E) with E = prod(tile); a token's slot is
    j*E plus its rank among its tile's tokens in tile-contiguous order.
    """
    E = tile[0] * tile[1] * tile[2]
    tid = token_tile_ids(T, Y, X, tile)
    order = tile_order(T, Y, X, tile)
    occ = occupancy(T, Y, X, tile)
    tile_start = np.concatenate([[0], np.cumsum(occ)[:-1]])   # position of each tile's first token
    pos = np.empty(len(tid), dtype=np.int64)
    pos[order] = np.arange(len(tid))                          # position of each token in the order
    return tid * E + (pos - tile_start[tid])


def tile_coords(T: int, Y: int, X: int, tile=TILE) -> np.ndarray:
    """(a, b, c) tile coordinates of every tile id j, int64 [Nt, 3]."""
    nt, ny, nx = tile_counts(T, Y, X, tile)
    a, b, c = np.meshgrid(np.arange(nt), np.arange(ny), np.arange(nx), indexing="ij")
    return np.stack([a.reshape(-1), b.reshape(-1), c.reshape(-1)], axis=1)
