"""Query pruning and the reconstruction of pruned positions.

Follows the "bsa_attn" page.  Its introduction says the method sparsifies
queries by pruning redundant tokens in each block, as well as key-value
blocks.  Its forward prunes the query blocks at a keep ratio (returning the
kept queries, their indices and the kept count), selects key-value blocks
from the kept queries, runs the sparse attention with the kept queries only,
and restores full block length from the sparse output, the kept indices and
the block size alone.

The page shows those calls but not their bodies.  Readings taken (each is
the plainest rule the calls and their arguments support):
  P1 kept count: a tile with n valid tokens keeps
     c = min(n, max(1, floor(ratio * n))) of them, ratio in (0, 1] (the
     floor-then-clamp rule the pages use to turn a ratio into a count).
  P2 which tokens: the least redundant ones.  A token is redundant when it
     points the way its tile's mean query points, so each valid token r
     scores cos(q_r, m), m the mean of the tile's valid queries (the cosine
     is 0 when either vector is zero), and the c lowest scores are kept,
     ties to the lower in-tile index.
  P3 selection: the kept queries' mean replaces the tile's pooled query in
     the block scores (the selection takes the pruned queries); keys are
     pooled as before.
  P4 attention: only kept rows attend, over the selected tiles' valid keys.
  P5 reconstruction: a kept row's output returns to its position; pruned
     and pad positions are +0.0 (the reconstruction sees only the sparse
     output, the kept indices and the block size, so it has nothing else to
     put there).

Everything is float64 except the pooled vectors (float32, as in select.py).
Test infrastructure only; shares no code with the GPU path.
"""
from __future__ import annotations

import math

import numpy as np

from . import attention, geometry, select


def kept_count(n: int, ratio: float) -> int:
    """Tokens kept of a tile with n valid tokens (reading P1)."""
    if not (0.0 < ratio <= 1.0):
        raise ValueError(f"keep ratio {ratio} outside (0, 1]")
    if n <= 0:
        return 0
    return min(n, max(1, math.floor(ratio * n)))


def redundancy(q: np.ndarray) -> np.ndarray:
    """cos(q_r, mean of the rows) for every row r of one tile's valid queries [n, D]."""
    q = q.astype(np.float64)
    m = q.mean(axis=0)
    dots = q @ m
    norms = np.linalg.norm(q, axis=1) * np.linalg.norm(m)
    out = np.zeros(len(q))
    nz = norms > 0
    out[nz] = dots[nz] / norms[nz]
    return out


def keep_mask(qt: np.ndarray, T: int, Y: int, X: int, ratio: float,
              tile=geometry.TILE) -> np.ndarray:
    """Kept query slots: bool [B, H, Nt, E], E the tile's slot count (readings
    P1, P2).

    qt: tile-ordered [B, Lpad, H, D] in the slot order of `tile`.  Slot r of
    tile j is kept when it is a valid token and among the kept_count(n_j)
    lowest redundancy scores of its tile (stable order: ties go to the lower
    slot).
    """
    B, lpad, H, _ = qt.shape
    E = geometry.tile_elems(tile)
    occ = geometry.occupancy(T, Y, X, tile)
    out = np.zeros((B, H, len(occ), E), dtype=bool)
    for b in range(B):
        for h in range(H):
            for j, n in enumerate(occ):
                c = kept_count(int(n), ratio)
                score = redundancy(qt[b, j * E:j * E + n, h])
                order = np.argsort(score, kind="stable")
                out[b, h, j, order[:c]] = True
    return out


def score_gap(qt: np.ndarray, T: int, Y: int, X: int, ratio: float,
              tile=geometry.TILE) -> np.ndarray:
    """Per tile, the lowest pruned minus the highest kept redundancy score
    (+inf when nothing is pruned): float64 [B, H, Nt].  A small gap means a
    near-tie at the keep boundary."""
    B, lpad, H, _ = qt.shape
    E = geometry.tile_elems(tile)
    occ = geometry.occupancy(T, Y, X, tile)
    out = np.full((B, H, len(occ)), np.inf)
    for b in range(B):
        for h in range(H):
            for j, n in enumerate(occ):
                c = kept_count(int(n), ratio)
                if c < n:
                    s = np.sort(redundancy(qt[b, j * E:j * E + n, h]))
                    out[b, h, j] = s[c] - s[c - 1]
    return out


def pool_kept(qt: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """Mean of each tile's kept query rows (reading P3): float32 [B, H, Nt, D]
    (float64 sum, one rounding).  The tile's slot count is keep's last axis."""
    B, lpad, H, D = qt.shape
    E = keep.shape[3]
    nt = keep.shape[2]
    out = np.zeros((B, H, nt, D), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            for j in range(nt):
                rows = np.nonzero(keep[b, h, j])[0]
                if len(rows):
                    x = qt[b, j * E + rows, h].astype(np.float64)
                    out[b, h, j] = (x.sum(axis=0) / len(rows)).astype(np.float32)
    return out


def pruned_attention(qt, kt, vt, mask, keep, T, Y, X, scale=None, rows=None,
                     tile=geometry.TILE):
    """Attention of the kept query rows, reconstructed to full tile length
    (readings P4, P5): (out float64 [B, Lpad, H, D], lse float64 [B, H, Lpad]);
    pruned and pad rows are 0 with lse -inf."""
    out, lse = attention.block_sparse_attention(qt, kt, vt, mask, T, Y, X, scale, rows, tile)
    B, lpad, H, _ = qt.shape
    kept_slots = keep.transpose(0, 2, 3, 1).reshape(B, lpad, H)   # [B, Nt*E, H]
    out[~kept_slots] = 0.0
    lse[~kept_slots.transpose(0, 2, 1)] = -np.inf
    return out, lse


def run(q_bits, k_bits, v_bits, T, Y, X, ratio, mode="cumulative", threshold=None,
        min_blocks=0, topk=None, rows=None, tile=geometry.TILE):
    """The pruned path: tile -> prune -> pool (kept Q, all K) -> score ->
    select (cumulative threshold, as the bsa_attn page's forward, or top-k)
    -> attention of kept rows -> reconstruct -> untile, for 64-token or
    128-token (`tile`) tiles."""
    from . import pipeline, tiling
    D = q_bits.shape[-1]
    qt = tiling.tile(pipeline.widen(q_bits), T, Y, X, tile)
    kt = tiling.tile(pipeline.widen(k_bits), T, Y, X, tile)
    vt = tiling.tile(pipeline.widen(v_bits), T, Y, X, tile)
    keep = keep_mask(qt, T, Y, X, ratio, tile)
    pq = pool_kept(qt, keep)
    pk = select.pool(kt, T, Y, X, tile)
    s = select.scores(pq, pk)
    if mode == "cumulative":
        mask = select.cumulative_mask(s, D, threshold, min_blocks)
    elif mode == "topk":
        mask = select.topk_mask(s, topk)
    else:
        raise ValueError(f"unknown mode {mode!r}")
    out_t, lse = pruned_attention(qt, kt, vt, mask, keep, T, Y, X, 1.0 / math.sqrt(D), rows, tile)
    return {"qt": qt, "kt": kt, "vt": vt, "keep": keep, "pq": pq, "pk": pk, "scores": s,
            "mask": mask, "out_tiled": out_t, "lse": lse,
            "out": tiling.untile(out_t, T, Y, X, tile)}
