"""The whole path on the CPU: tile -> pool -> score -> select -> CSR -> attend -> untile.

Follows the order of the "bsa_attn" page (preprocess_qkv, forward,
postprocess_output) with the coarse stage of the "sla" page's get_block_map
(top-k) or a sliding-tile window of the "STA_configuration" page (STA).
Inputs are bf16 bits (uint16 [B, L, H, D]); they are widened exactly to
float64 before any arithmetic.
"""
from __future__ import annotations

import math

import numpy as np

from . import attention, geometry, select, tiling


def widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bits -> float64 values (exact)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def block_mask(qt, kt, T, Y, X, mode, topk=None, windows=None, tile=geometry.TILE):
    """Pooled vectors, scores and the block mask of the coarse stage."""
    B, _, H, _ = qt.shape
    if mode == "topk":
        pq = select.pool(qt, T, Y, X, tile)
        pk = select.pool(kt, T, Y, X, tile)
        s = select.scores(pq, pk)
        return {"pq": pq, "pk": pk, "scores": s, "mask": select.topk_mask(s, topk)}
    if mode == "sta":
        return {"mask": select.sta_mask(T, Y, X, np.asarray(windows), B, tile)}
    raise ValueError(f"unknown mode {mode!r}")


def run(q_bits, k_bits, v_bits, T, Y, X, mode, topk=None, windows=None, rows=None,
        tile=geometry.TILE):
    """Run the path; rows limits attention to a list of (b, h, i) query tiles.
    ``tile`` is the tile shape (geometry.TILE_SHAPES)."""
    D = q_bits.shape[-1]
    qt = tiling.tile(widen(q_bits), T, Y, X, tile)
    kt = tiling.tile(widen(k_bits), T, Y, X, tile)
    vt = tiling.tile(widen(v_bits), T, Y, X, tile)
    res = block_mask(qt, kt, T, Y, X, mode, topk, windows, tile)
    res["row_ptr"], res["col_idx"] = select.mask_to_csr(res["mask"])
    out_t, lse = attention.block_sparse_attention(qt, kt, vt, res["mask"], T, Y, X,
                                                  1.0 / math.sqrt(D), rows, tile)
    res.update(qt=qt, kt=kt, vt=vt, out_tiled=out_t, lse=lse,
               out=tiling.untile(out_t, T, Y, X, tile))
    return res
