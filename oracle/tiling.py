"""Raster order <-> zero-padded tile order for [B, L, H, D] tensors.

Follows the "bsa_attn" page (preprocess_qkv gathers tokens into tile order
along the sequence axis; postprocess_output applies the reverse permutation)
and the "video_sparse_attn_h3" page (tile(): rows are scattered into a padded
tile buffer whose pad positions stay zero; the sequence length must match the
geometry, else ValueError).
"""
from __future__ import annotations

import numpy as np

from . import geometry


def tile(x: np.ndarray, T: int, Y: int, X: int, tile=geometry.TILE) -> np.ndarray:
    """[B, L, H, D] raster -> [B, Lpad, H, D] tile order, pad slots zero."""
    B, L, H, D = x.shape
    if L != T * Y * X:
        raise ValueError(f"sequence length {L} does not match grid {T}x{Y}x{X}")
    lpad = geometry.padded_len(T, Y, X, tile)
    out = np.zeros((B, lpad, H, D), dtype=x.dtype)
    out[:, geometry.token_slots(T, Y, X, tile)] = x
    return out


def untile(xt: np.ndarray, T: int, Y: int, X: int, tile=geometry.TILE) -> np.ndarray:
    """[B, Lpad, H, D] tile order -> [B, L, H, D] raster; pad slots dropped."""
    if xt.shape[1] != geometry.padded_len(T, Y, X, tile):
        raise ValueError("padded length does not match the grid")
    return xt[:, geometry.token_slots(T, Y, X, tile)]
