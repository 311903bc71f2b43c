"""Masked softmax attention over selected tiles, and a dense brute force.

Follows the "bsa_attn" page: attention is bidirectional (no causal mask),
query/key/value share one head count (no grouped-query attention), the
softmax scale is 1/sqrt(d), and the sparse attention of a query block runs
over the key/value blocks its block mask keeps (_compute_sparse_attention on
tile-ordered [B, L, H, D] tensors).  Inside a tile only the n_j valid tokens
take part; padded query rows produce zero output (the padded buffer keeps
pad positions zero, "video_sparse_attn_h3" page, tile()).

Everything is float64.  The log-sum-exp of a valid row is the natural log of
the softmax denominator of the scaled scores; a padded row has lse = -inf.

The backward pass (gradients of sum(dO * O) with respect to Q, K and V) is
the chain rule through the same masked softmax; the bsa_attn page notes the
method targets training, and the video_sparse_attn_h3 page's tile() keeps
a gradient route through its gather.
"""
from __future__ import annotations

import math

import numpy as np

from . import geometry


def tile_attention(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float):
    """softmax(q keys^T * scale) vals for one query block; returns (o, lse)."""
    s = (q @ keys.T) * scale
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ vals) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def block_sparse_attention(qt, kt, vt, mask, T, Y, X, scale=None, rows=None, tile=geometry.TILE):
    """Attention of tile-ordered [B, Lpad, H, D] tensors under a block mask.

    mask: bool [B, H, Nt, Nt].  rows: optional list of (b, h, i) query tiles
    to compute; others are left zero (lse -inf).  Returns (out, lse) with out
    float64 [B, Lpad, H, D] and lse float64 [B, H, Lpad].
    """
    B, lpad, H, D = qt.shape
    E = geometry.tile_elems(tile)
    occ = geometry.occupancy(T, Y, X, tile)
    nt = len(occ)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.zeros((B, lpad, H, D), dtype=np.float64)
    lse = np.full((B, H, lpad), -np.inf, dtype=np.float64)
    if rows is None:
        rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(nt)]
    for b, h, i in rows:
        sel = np.nonzero(mask[b, h, i])[0]
        if len(sel) == 0:
            continue
        keys = np.concatenate([kt[b, j * E:j * E + occ[j], h, :] for j in sel]).astype(np.float64)
        vals = np.concatenate([vt[b, j * E:j * E + occ[j], h, :] for j in sel]).astype(np.float64)
        q = qt[b, i * E:i * E + occ[i], h, :].astype(np.float64)
        o, l = tile_attention(q, keys, vals, scale)
        out[b, i * E:i * E + occ[i], h, :] = o
        lse[b, h, i * E:i * E + occ[i]] = l
    return out, lse


def tile_attention_backward(q, keys, vals, do, scale: float):
    """Gradients of sum(do * o) for o = softmax(q keys^T * scale) vals.

    The chain rule through the softmax, written out: with P the softmax
    probabilities and dP = do vals^T, the score gradient is
    dS = P * (dP - rowsum(do * o)) (rowsum(do * o) = rowsum(P * dP)), so
    dq = dS keys * scale, dkeys = dS^T q * scale and dvals = P^T do.
    Returns (dq, dkeys, dvals).
    """
    s = (q @ keys.T) * scale
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    o = p @ vals
    dp = do @ vals.T
    delta = (do * o).sum(axis=1, keepdims=True)
    ds = p * (dp - delta)
    return (ds @ keys) * scale, (ds.T @ q) * scale, p.T @ do


def block_sparse_attention_backward(qt, kt, vt, dot, mask, T, Y, X, scale=None, tile=geometry.TILE):
    """Gradients of the block-sparse attention of tile-ordered tensors.

    For the loss sum(dot * out) with out = block_sparse_attention(...):
    query tile i of head h attends over the valid tokens of the key tiles
    mask[b, h, i] keeps, so its rows receive dq from those keys, and each
    kept key/value tile receives dk, dv from every query tile that keeps it.
    Padded slots (query or key) get zero gradient.  Inputs [B, Lpad, H, D]
    in the slot order of `tile` (4x4x4 or 4x4x8 tokens); returns float64
    (dq, dk, dv) of that shape.
    """
    B, lpad, H, D = qt.shape
    E = geometry.tile_elems(tile)
    occ = geometry.occupancy(T, Y, X, tile)
    nt = len(occ)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = np.zeros((B, lpad, H, D), dtype=np.float64)
    dk = np.zeros_like(dq)
    dv = np.zeros_like(dq)
    for b in range(B):
        for h in range(H):
            for i in range(nt):
                sel = np.nonzero(mask[b, h, i])[0]
                if len(sel) == 0:
                    continue
                keys = np.concatenate([kt[b, j * E:j * E + occ[j], h, :] for j in sel]).astype(np.float64)
                vals = np.concatenate([vt[b, j * E:j * E + occ[j], h, :] for j in sel]).astype(np.float64)
                rows = slice(i * E, i * E + occ[i])
                gq, gk, gv = tile_attention_backward(qt[b, rows, h, :].astype(np.float64), keys, vals,
                                                     dot[b, rows, h, :].astype(np.float64), scale)
                dq[b, rows, h, :] = gq
                at = 0
                for j in sel:
                    cols = slice(j * E, j * E + occ[j])
                    dk[b, cols, h, :] += gk[at:at + occ[j]]
                    dv[b, cols, h, :] += gv[at:at + occ[j]]
                    at += occ[j]
    return dq, dk, dv


def dense_masked_attention(q, k, v, mask, T, Y, X, scale=None, tile=geometry.TILE):
    """Brute force in raster order with an explicit L x L 0/-inf token mask.

    q, k, v: [B, L, H, D]; mask: bool block mask [B, H, Nt, Nt].  The token
    mask lets query token l see key token l' iff mask[tile(l), tile(l')].
    Returns (out float64 [B, L, H, D], lse float64 [B, H, L]).
    """
    B, L, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    tid = geometry.token_tile_ids(T, Y, X, tile)
    out = np.empty((B, L, H, D), dtype=np.float64)
    lse = np.empty((B, H, L), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            tokmask = np.where(mask[b, h][tid][:, tid], 0.0, -np.inf)
            s = (q[b, :, h].astype(np.float64) @ k[b, :, h].astype(np.float64).T) * scale + tokmask
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            l = p.sum(axis=1, keepdims=True)
            out[b, :, h] = (p @ v[b, :, h].astype(np.float64)) / l
            lse[b, h] = (m + np.log(l))[:, 0]
    return out, lse
