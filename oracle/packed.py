"""Packed multi-region sequences: dense segments and video regions in one sequence.

Follows the "video_sparse_attn_h3" page, build(): the packed sequence lists,
in packed order, dense segments (a row count; empty ones are dropped) and
video regions (a raw latent shape (t, h, w), which must be a positive
multiple of the patch size and becomes a token grid of (t, h, w) / patch).
At least one video region is required; the last region is the generated
video and follows the sparsity; every earlier region is a reference video
that keeps ref_keep_rate of its tiles (required when there is more than one
region); the compete mode supports only the generated region; a sparsity of
0 keeps every region dense.  The geometry it builds has a prefix of tiles,
video tiles, per-region tile spans and per-tile valid counts; the page shows
the call, not the body.

Readings taken (R24; parity is pinned to them, not to the page):
  G1 tiles: a dense segment of n rows is cut into ceil(n/64) tiles of
     consecutive rows (the last one partial); a video region's token grid is
     cut into 4x4x4 tiles exactly as a single grid (tile order time-major,
     valid tokens first inside a tile).
  G2 tile order: every dense segment's tiles first (the prefix), in packed
     order, then each video region's tiles, region by region in packed
     order; a region's tiles form its span [start, end).
  G3 slots: tile j owns slots [64 j, 64 j + 64); its valid tokens come first.
  G4 selection, exempt mode (the default): a prefix query tile attends every
     tile; a video query tile attends every prefix tile and, in each video
     span r, the k_r key tiles of that span with the highest pooled score
     (ties to the lower index), k_r = min(n_r, max(1, floor(keep_r * n_r)))
     with keep_r = 1 - sparsity_r (the floor-then-clamp rule of the top-k
     ratio): ref_keep_rate for reference regions, 1 - sparsity for the last.
     A sparsity of 0 or below keeps every tile.
  G5 compete mode (one video region only): every query tile keeps the
     min(Nt, max(1, floor((1 - sparsity) * Nt))) best key tiles of the whole
     packed sequence, prefix tiles competing with video tiles.
  G6 pooling, scores and attention as for a single grid (per-tile means of
     the valid rows, unscaled pooled dot products, softmax at 1/sqrt(D) over
     the valid tokens of the selected tiles, pad rows zero).

Test infrastructure only; shares no code with the GPU path.
"""
from __future__ import annotations

import math

import numpy as np

from . import geometry

E = geometry.TILE_ELEMS


def token_segments(packed_segments, patch=(1, 1, 1)):
    """Packed segments -> token segments: ints (dense rows, empty ones dropped)
    and (T, Y, X) token grids (latent shape / patch).  Raises ValueError as
    the page's build() does."""
    out = []
    for seg in packed_segments:
        if isinstance(seg, tuple):
            if any(int(v) <= 0 or int(v) % p for v, p in zip(seg, patch)):
                raise ValueError(f"region {seg} is not a positive multiple of patch {patch}")
            out.append(tuple(int(v) // p for v, p in zip(seg, patch)))
        elif int(seg) > 0:
            out.append(int(seg))
    if not any(isinstance(s, tuple) for s in out):
        raise ValueError("at least one video region is required")
    return out


def layout(segments):
    """Tile layout of token segments (readings G1-G3).

    Returns a dict: ``occ`` int64 [Nt] valid tokens per tile; ``slot_token``
    int64 [Nt*64] packed token of each slot (-1 for pads); ``num_prefix``;
    ``spans`` list of (start, end) tile ranges of the video regions in packed
    order; ``L`` the packed length.
    """
    offsets, L = [], 0
    for s in segments:
        offsets.append(L)
        L += math.prod(s) if isinstance(s, tuple) else s
    tiles = []          # (token ids of the tile, in slot order)
    for s, off in zip(segments, offsets):      # prefix: dense segments first
        if isinstance(s, tuple):
            continue
        for a in range(0, s, E):
            tiles.append(np.arange(off + a, off + min(s, a + E)))
    num_prefix = len(tiles)
    spans = []
    for s, off in zip(segments, offsets):
        if not isinstance(s, tuple):
            continue
        T, Y, X = s
        start = len(tiles)
        slots = geometry.token_slots(T, Y, X)
        nt = geometry.num_tiles(T, Y, X)
        order = np.argsort(slots, kind="stable")
        tile_of = slots[order] // E
        for j in range(nt):
            tiles.append(off + order[tile_of == j])
        spans.append((start, start + nt))
    occ = np.array([len(t) for t in tiles], dtype=np.int64)
    slot_token = np.full(len(tiles) * E, -1, dtype=np.int64)
    for j, t in enumerate(tiles):
        slot_token[j * E:j * E + len(t)] = t
    return {"occ": occ, "slot_token": slot_token, "num_prefix": num_prefix, "spans": spans, "L": L}


def tile(x, lay):
    """[B, L, H, D] packed -> [B, Nt*64, H, D] tile order, pads zero."""
    B, L, H, D = x.shape
    if L != lay["L"]:
        raise ValueError(f"sequence length {L} does not match the packed length {lay['L']}")
    out = np.zeros((B, len(lay["slot_token"]), H, D), dtype=x.dtype)
    valid = lay["slot_token"] >= 0
    out[:, valid] = x[:, lay["slot_token"][valid]]
    return out


def untile(xt, lay):
    """Inverse of tile over valid slots."""
    B, _, H, D = xt.shape
    out = np.zeros((B, lay["L"], H, D), dtype=xt.dtype)
    valid = lay["slot_token"] >= 0
    out[:, lay["slot_token"][valid]] = xt[:, valid]
    return out


def pool(xt, lay):
    """Mean of the valid rows of every tile: float32 [B, H, Nt, D] (float64 sum)."""
    B, _, H, D = xt.shape
    occ = lay["occ"]
    out = np.empty((B, H, len(occ), D), dtype=np.float32)
    for j, n in enumerate(occ):
        out[:, :, j, :] = (xt[:, j * E:j * E + n].astype(np.float64).sum(axis=1) / n).astype(np.float32)
    return out


def keep_count(n: int, keep: float) -> int:
    """Tiles kept of a span of n tiles at keep fraction `keep` (reading G4)."""
    return min(n, max(1, math.floor(keep * n)))


def span_keeps(lay, sparsity: float, ref_keep_rate=None):
    """keep fraction of each video span (reading G4): reference regions keep
    ref_keep_rate, the last region 1 - sparsity; sparsity <= 0 keeps all."""
    R = len(lay["spans"])
    if R > 1 and ref_keep_rate is None:
        raise ValueError("reference regions need ref_keep_rate")
    if sparsity <= 0.0:
        return [1.0] * R
    refs = [float(ref_keep_rate)] * (R - 1) if R > 1 else []
    return refs + [1.0 - float(sparsity)]


def select_mask(scores, lay, sparsity: float, ref_keep_rate=None, exempt: bool = True):
    """Block mask [B, H, Nt, Nt] of the packed selection (readings G4, G5)."""
    B, H, nt, _ = scores.shape
    P = lay["num_prefix"]
    mask = np.zeros(scores.shape, dtype=bool)
    if not exempt:
        if len(lay["spans"]) != 1:
            raise ValueError("compete mode supports only the generated-video region")
        k = nt if sparsity <= 0.0 else keep_count(nt, 1.0 - float(sparsity))
        order = np.argsort(-scores, axis=-1, kind="stable")
        np.put_along_axis(mask, order[..., :k], True, axis=-1)
        return mask
    keeps = span_keeps(lay, sparsity, ref_keep_rate)
    mask[:, :, :P, :] = True                # prefix query tiles attend everything
    mask[:, :, P:, :P] = True               # video query tiles attend the whole prefix
    for (a, b), keep in zip(lay["spans"], keeps):
        k = keep_count(b - a, keep)
        sub = scores[:, :, P:, a:b]
        order = np.argsort(-sub, axis=-1, kind="stable")
        part = np.zeros(sub.shape, dtype=bool)
        np.put_along_axis(part, order[..., :k], True, axis=-1)
        mask[:, :, P:, a:b] = part
    return mask


def attention(qt, kt, vt, mask, lay, scale=None, rows=None):
    """Masked softmax attention of tile-ordered tensors under a block mask,
    over the valid tokens of the selected tiles (float64); pads 0, lse -inf."""
    B, lpad, H, D = qt.shape
    occ = lay["occ"]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.zeros((B, lpad, H, D))
    lse = np.full((B, H, lpad), -np.inf)
    if rows is None:
        rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(len(occ))]
    for b, h, i in rows:
        sel = np.nonzero(mask[b, h, i])[0]
        keys = np.concatenate([kt[b, j * E:j * E + occ[j], h] for j in sel]).astype(np.float64)
        vals = np.concatenate([vt[b, j * E:j * E + occ[j], h] for j in sel]).astype(np.float64)
        q = qt[b, i * E:i * E + occ[i], h].astype(np.float64)
        s = q @ keys.T * scale
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        l = p.sum(axis=1, keepdims=True)
        out[b, i * E:i * E + occ[i], h] = p @ vals / l
        lse[b, h, i * E:i * E + occ[i]] = (m + np.log(l))[:, 0]
    return out, lse


def attention_backward(qt, kt, vt, dot, mask, lay, scale=None):
    """Gradients of sum(dot * out) for out = attention(qt, kt, vt, mask, lay)
    (float64, tile-ordered [B, Nt*64, H, D]): per query tile, the softmax
    chain rule over the valid tokens of its selected tiles
    (attention.tile_attention_backward), the key/value gradients summed over
    every query tile that selects them; pad slots get zero."""
    from .attention import tile_attention_backward
    B, lpad, H, D = qt.shape
    occ = lay["occ"]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq, dk, dv = (np.zeros((B, lpad, H, D)) for _ in range(3))
    for b in range(B):
        for h in range(H):
            for i in range(len(occ)):
                sel = np.nonzero(mask[b, h, i])[0]
                if len(sel) == 0:
                    continue
                keys = np.concatenate([kt[b, j * E:j * E + occ[j], h] for j in sel]).astype(np.float64)
                vals = np.concatenate([vt[b, j * E:j * E + occ[j], h] for j in sel]).astype(np.float64)
                rows = slice(i * E, i * E + occ[i])
                gq, gk, gv = tile_attention_backward(qt[b, rows, h].astype(np.float64), keys, vals,
                                                     dot[b, rows, h].astype(np.float64), scale)
                dq[b, rows, h] = gq
                at = 0
                for j in sel:
                    cols = slice(j * E, j * E + occ[j])
                    dk[b, cols, h] += gk[at:at + occ[j]]
                    dv[b, cols, h] += gv[at:at + occ[j]]
                    at += occ[j]
    return dq, dk, dv


def run(q, k, v, packed_segments, patch=(1, 1, 1), sparsity=0.9, ref_keep_rate=None,
        exempt=True, rows=None):
    """The packed path on float arrays [B, L, H, D]: geometry, tile, pool,
    score, select, attend, untile."""
    segs = token_segments(packed_segments, patch)
    lay = layout(segs)
    qt, kt, vt = (tile(x.astype(np.float64), lay) for x in (q, k, v))
    pq, pk = pool(qt, lay), pool(kt, lay)
    s = np.matmul(pq.astype(np.float64), np.swapaxes(pk.astype(np.float64), -1, -2))
    mask = select_mask(s, lay, sparsity, ref_keep_rate, exempt)
    out_t, lse = attention(qt, kt, vt, mask, lay, rows=rows)
    return {"layout": lay, "qt": qt, "kt": kt, "vt": vt, "pq": pq, "pk": pk, "scores": s,
            "mask": mask, "out_tiled": out_t, "lse": lse, "out": untile(out_t, lay)}
