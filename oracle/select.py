"""Coarse stage: per-tile mean pooling, pooled scores, block selection, CSR.

Follows:
  * "sla" page, get_block_map: Q and K are mean-pooled per block, the pooled
    score matrix is pooled_q @ pooled_k^T with no scale, and each query block
    keeps the top-k key blocks (topk = min(K, int(ratio*K)) when a ratio is
    given), scattered into a 0/1 block map.
  * "sla" page, mean_pool: one mean vector per block of the sequence axis.
  * "STA_configuration" page: a sliding-tile window is a triple of tile
    counts along (t, h, w); every query is charged prod(window) tiles and the
    full-grid window is full attention (select_best_mask_strategy's sparsity
    accounting).
  * "video_sparse_attn_h3" page: map_to_index turns the block mask into an
    index form consumed by the sparse kernel.

Readings taken where the pages are silent:
  * pooling divides by the tile's valid-token count n_j (a true per-tile
    mean) and the pooled vectors are float32 (float64 sum, one rounding);
  * the "smooth-k" shift (k minus its mean over L) is left out: it subtracts
    the same amount from every score of a row, so the selected set is
    unchanged in exact arithmetic;
  * ties in top-k go to the lower key-tile index; CSR columns are ascending;
  * STA windows are shifted (clamped centre) windows: a window of w tiles
    starting at clamp(a - floor(w/2), 0, n - w) on each axis, so every row
    holds exactly prod(window) tiles and the full-grid window is dense.
  * cumulative-threshold selection ("bsa_attn" page, forward: the key-value
    block selection takes a cumulative threshold and a minimum block count;
    the rule itself is not on the page): the pooled scores of a row, scaled
    by the attention's 1/sqrt(D), go through a softmax over key tiles; the
    tiles are taken in descending score order (ties to the lower index) and
    a row keeps the shortest such prefix whose probability mass reaches the
    threshold, but never fewer than min(min_blocks, Nt) tiles.
"""
from __future__ import annotations

import numpy as np

from . import geometry


def pool(xt: np.ndarray, T: int, Y: int, X: int, tile=geometry.TILE) -> np.ndarray:
    """Mean of the valid rows of every tile: [B, Lpad, H, D] -> f32 [B, H, Nt, D]."""
    B, lpad, H, D = xt.shape
    E = geometry.tile_elems(tile)
    occ = geometry.occupancy(T, Y, X, tile)
    out = np.empty((B, H, len(occ), D), dtype=np.float32)
    for j, n in enumerate(occ):
        rows = xt[:, j * E:j * E + n].astype(np.float64)     # [B, n, H, D]
        out[:, :, j, :] = (rows.sum(axis=1) / n).astype(np.float32)
    return out


def scores(pq: np.ndarray, pk: np.ndarray) -> np.ndarray:
    """Pooled score matrix S = Pq Pk^T (float64, no scale): [B, H, Nt, Nt]."""
    return np.matmul(pq.astype(np.float64), np.swapaxes(pk.astype(np.float64), -1, -2))


def topk_mask(s: np.ndarray, k: int) -> np.ndarray:
    """Keep the k largest scores of each row; ties go to the lower index."""
    nt = s.shape[-1]
    if not 1 <= k <= nt:
        raise ValueError(f"k={k} outside [1, {nt}]")
    order = np.argsort(-s, axis=-1, kind="stable")
    mask = np.zeros(s.shape, dtype=bool)
    np.put_along_axis(mask, order[..., :k], True, axis=-1)
    return mask


def boundary_gap(s: np.ndarray, k: int) -> np.ndarray:
    """S_(k) - S_(k+1) per row (k-th and (k+1)-th largest); +inf when k = Nt."""
    nt = s.shape[-1]
    desc = -np.sort(-s, axis=-1)
    if k >= nt:
        return np.full(s.shape[:-1], np.inf)
    return desc[..., k - 1] - desc[..., k]


def kth_values(s: np.ndarray, k: int):
    """(S_(k), S_(k+1)) per row; S_(k+1) = -inf when k = Nt."""
    nt = s.shape[-1]
    desc = -np.sort(-s, axis=-1)
    upper = desc[..., k - 1]
    lower = desc[..., k] if k < nt else np.full(s.shape[:-1], -np.inf)
    return upper, lower


def cumulative_counts(s: np.ndarray, D: int, threshold: float, min_blocks: int = 0) -> np.ndarray:
    """Tiles kept per row by the cumulative-threshold rule: int64 [...].

    p = softmax(S / sqrt(D)) over the row's key tiles (float64); with the
    tiles in descending score order, the count is the first prefix length
    whose summed p reaches `threshold` (Nt if none does, which only rounding
    can cause), raised to min(min_blocks, Nt).
    """
    if not (0.0 < threshold <= 1.0):
        raise ValueError(f"threshold {threshold} outside (0, 1]")
    if min_blocks < 0:
        raise ValueError(f"min_blocks {min_blocks} < 0")
    nt = s.shape[-1]
    z = s.astype(np.float64) / np.sqrt(float(D))
    p = np.exp(z - z.max(axis=-1, keepdims=True))
    p = p / p.sum(axis=-1, keepdims=True)
    order = np.argsort(-s, axis=-1, kind="stable")
    mass = np.cumsum(np.take_along_axis(p, order, axis=-1), axis=-1)
    counts = np.minimum((mass < threshold).sum(axis=-1) + 1, nt)
    return np.maximum(counts, min(min_blocks, nt))


def prefix_mask(s: np.ndarray, counts: np.ndarray) -> np.ndarray:
    """Keep the counts[r] best-scored tiles of every row r; ties to the lower index."""
    nt = s.shape[-1]
    order = np.argsort(-s, axis=-1, kind="stable")
    rank = np.empty_like(order)
    np.put_along_axis(rank, order, np.broadcast_to(np.arange(nt), order.shape), axis=-1)
    return rank < np.asarray(counts)[..., None]


def cumulative_mask(s: np.ndarray, D: int, threshold: float, min_blocks: int = 0) -> np.ndarray:
    """Block mask of the cumulative-threshold selection: bool, shape of s."""
    return prefix_mask(s, cumulative_counts(s, D, threshold, min_blocks))


def cumulative_masses(s: np.ndarray, D: int) -> np.ndarray:
    """Probability mass of the top-c prefix of every row, c = 1..Nt (float64)."""
    z = s.astype(np.float64) / np.sqrt(float(D))
    p = np.exp(z - z.max(axis=-1, keepdims=True))
    p = p / p.sum(axis=-1, keepdims=True)
    order = np.argsort(-s, axis=-1, kind="stable")
    return np.cumsum(np.take_along_axis(p, order, axis=-1), axis=-1)


def topk_from_ratio(ratio: float, nt: int) -> int:
    """k for a density ratio, as the pages derive it: min(Nt, int(ratio*Nt))."""
    return min(nt, int(ratio * nt))


def sta_window_start(a: int, w: int, n: int) -> int:
    """First tile of a w-tile window around tile a on an axis of n tiles."""
    return min(max(a - w // 2, 0), n - w)


def sta_mask(T: int, Y: int, X: int, windows: np.ndarray, B: int, tile=geometry.TILE) -> np.ndarray:
    """Block mask of per-head sliding tile windows: bool [B, H, Nt, Nt]."""
    n = geometry.tile_counts(T, Y, X, tile)
    coords = geometry.tile_coords(T, Y, X, tile)
    nt = len(coords)
    H = len(windows)
    mask = np.zeros((H, nt, nt), dtype=bool)
    for h in range(H):
        w = [int(v) for v in windows[h]]
        for ax in range(3):
            if not 1 <= w[ax] <= n[ax]:
                raise ValueError(f"head {h}: window {w} outside grid {n}")
        for i in range(nt):
            keep = np.ones(nt, dtype=bool)
            for ax in range(3):
                st = sta_window_start(int(coords[i, ax]), w[ax], n[ax])
                keep &= (coords[:, ax] >= st) & (coords[:, ax] < st + w[ax])
            mask[h, i] = keep
    return np.broadcast_to(mask[None], (B, H, nt, nt)).copy()


def mask_to_csr(mask: np.ndarray):
    """Block mask [B, H, Nt, Nt] -> (row_ptr int32 [B*H*Nt+1], col_idx int32).

    Row r = (b*H + h)*Nt + i lists the selected key tiles of query tile i of
    head h in batch b, in ascending order.
    """
    rows = mask.reshape(-1, mask.shape[-1])
    counts = rows.sum(axis=1)
    row_ptr = np.zeros(len(rows) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.nonzero(rows)[1]
    return row_ptr.astype(np.int32), col_idx.astype(np.int32)
