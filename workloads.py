"""Seeded synthetic workloads for block-sparse tiled video attention.

This module only makes inputs: it draws seeded random tensors with the shapes
and value structure of the five workloads, rounds them once to bfloat16, and
hands out the raw bf16 bits (``uint16``).  Both the CPU oracle (``oracle/``)
and the HIP path consume exactly these bits.  Nothing here computes any step
of the method (no tile permutation, no pooling, no selection, no attention):
the only geometry used is "which 4x4x4 cell of the latent grid does a token
fall in", as coordinates, to place the per-cell structure terms.

Recipe (one per workload, seed = workload index 0..4):
  * Q, K, V ~ N(0, 1) float32 of shape [B, L, H, D] in raster token order
    (token l = (t*Y + y)*X + x), drawn from counter-indexed PCG64 child
    streams ``SeedSequence(seed, spawn_key=(tensor, chunk))`` so that chunks
    can be drawn in parallel threads with a result independent of threading.
  * structure terms (added to float32 Q and K before the bf16 rounding):
      - lowrank: per head, A ~ N(0,1) [cells, 4], Bm ~ N(0,1) [D, 4];
        G = A Bm^T scaled to std 0.5; G of the token's 4x4x4 cell is added to
        both Q and K (a shared per-cell low-rank bias).
      - smooth: per head, white noise [T, Y, X, D] blurred by a 3-D Gaussian
        (sigma 2 tokens along T, Y, X; none along D; reflect borders,
        truncate 4), each channel scaled to unit std, times 0.5, added to
        both Q and K.
  * STA windows (sta workloads): per head one of (1,3,3), (3,3,3), (3,5,5)
    tiles, index drawn uniformly from a stream of its own; shared by all
    batch items.
  * packed sequences (make_packed_inputs): Q, K, V ~ N(0, 1) over the packed
    length; "smooth" adds the smooth term above to each video region (a
    field of its own per region), none to dense segments.
  * every tensor is rounded once to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TILE = (4, 4, 4)
STA_CANDIDATES = ((1, 3, 3), (3, 3, 3), (3, 5, 5))
_CHUNK = 1 << 22  # elements per independent random stream
_THREADS = 8


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    B: int
    H: int
    D: int
    T: int
    Y: int
    X: int
    mode: str          # "topk" or "sta"
    topk: int = 0
    structure: str = "none"   # "none", "lowrank", "smooth"

    @property
    def L(self) -> int:
        return self.T * self.Y * self.X

    @property
    def seed(self) -> int:
        return self.index

    def describe(self) -> dict:
        d = dataclasses.asdict(self)
        d["L"] = self.L
        return d


WORKLOADS = {
    "c1": Workload("c1", 0, 1, 2, 64, 8, 8, 8, "topk", 2),
    "c2": Workload("c2", 1, 1, 12, 128, 16, 32, 32, "topk", 32, "lowrank"),
    "c3": Workload("c3", 2, 1, 40, 128, 20, 48, 80, "topk", 120, "smooth"),
    "c4": Workload("c4", 3, 1, 40, 128, 21, 30, 52, "topk", 62),
    "c5": Workload("c5", 4, 2, 24, 128, 16, 48, 80, "sta"),
}


def custom(name, B, H, D, T, Y, X, mode="topk", topk=1, structure="none",
           seed=1000) -> Workload:
    """A workload of arbitrary shape (used for small and ragged test cases)."""
    return Workload(name, seed, B, H, D, T, Y, X, mode, topk, structure)


def _pool():
    return ThreadPoolExecutor(_THREADS)


def _normal(shape, seed: int, stream: int) -> np.ndarray:
    """float32 N(0,1) of ``shape`` from counter-indexed child streams."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nchunks = max(1, (n + _CHUNK - 1) // _CHUNK)

    def fill(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        ss = np.random.SeedSequence(seed, spawn_key=(stream, c))
        out[lo:hi] = np.random.Generator(np.random.PCG64(ss)).standard_normal(
            hi - lo, dtype=np.float32)

    with _pool() as ex:
        list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    step = 1 << 24

    def conv(c):
        u = flat[c * step:(c + 1) * step].view(np.uint32)
        r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        out[c * step:(c + 1) * step] = r.astype(np.uint16)

    with _pool() as ex:
        list(ex.map(conv, range((flat.size + step - 1) // step)))
    return out.reshape(x.shape)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to float32."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _cell_coords(w: Workload):
    """Per raster token, the coordinates of its 4x4x4 cell (generator-side)."""
    t = np.arange(w.T) // TILE[0]
    y = np.arange(w.Y) // TILE[1]
    x = np.arange(w.X) // TILE[2]
    return t, y, x


def _add_lowrank(w: Workload, q, k):
    nt = math.ceil(w.T / TILE[0])
    ny = math.ceil(w.Y / TILE[1])
    nx = math.ceil(w.X / TILE[2])
    ct, cy, cx = _cell_coords(w)
    for h in range(w.H):
        a = _normal((nt, ny, nx, 4), w.seed, 100 + 2 * h)
        bm = _normal((w.D, 4), w.seed, 101 + 2 * h)
        g = (a.reshape(-1, 4).astype(np.float64) @ bm.astype(np.float64).T)
        g = (g * (0.5 / g.std())).astype(np.float32).reshape(nt, ny, nx, w.D)
        per_tok = g[ct][:, cy][:, :, cx].reshape(w.L, w.D)
        q[:, :, h, :] += per_tok[None]
        k[:, :, h, :] += per_tok[None]


def _add_smooth(w: Workload, q, k):
    from scipy import ndimage
    for h in range(w.H):
        noise = _normal((w.T, w.Y, w.X, w.D), w.seed, 100 + h)
        sm = np.empty_like(noise)
        parts = 8
        step = (w.D + parts - 1) // parts

        def blur(c):
            sl = slice(c * step, min(w.D, (c + 1) * step))
            if sl.start < sl.stop:
                sm[..., sl] = ndimage.gaussian_filter(
                    noise[..., sl], sigma=(2, 2, 2, 0), mode="reflect", truncate=4.0)

        with _pool() as ex:
            list(ex.map(blur, range(parts)))
        sm = sm.reshape(w.L, w.D)
        sm *= (0.5 / sm.std(axis=0, dtype=np.float64)).astype(np.float32)[None]
        q[:, :, h, :] += sm[None]
        k[:, :, h, :] += sm[None]


def make_packed_inputs(B, H, D, token_segments, seed, structure="none"):
    """bf16 bits q, k, v [B, L, H, D] of a packed sequence.  ``token_segments``
    lists dense segments (ints, rows) and video regions ((T, Y, X) token
    grids) in packed order; L is their total length.  Q, K, V ~ N(0, 1) as in
    make_inputs; with ``structure`` "smooth" each video region r gets the
    smooth term of a (T, Y, X) grid drawn with seed 1000 * seed + r + 1 (its
    own fields), dense segments none."""
    L = sum(int(np.prod(s)) if isinstance(s, tuple) else int(s) for s in token_segments)
    shape = (B, L, H, D)
    q = _normal(shape, seed, 0)
    k = _normal(shape, seed, 1)
    v = _normal(shape, seed, 2)
    if structure == "smooth":
        off, r = 0, 0
        for s in token_segments:
            n = int(np.prod(s)) if isinstance(s, tuple) else int(s)
            if isinstance(s, tuple):
                w = Workload("region", 1000 * seed + r + 1, B, H, D, *s, "topk", 1, "smooth")
                _add_smooth(w, q[:, off:off + n], k[:, off:off + n])
                r += 1
            off += n
    elif structure != "none":
        raise ValueError(f"unknown structure {structure!r}")
    return {"q": bf16_bits(q), "k": bf16_bits(k), "v": bf16_bits(v)}


def sta_windows(w: Workload) -> np.ndarray:
    """Per-head STA window (tiles along T, Y, X), int32 [H, 3]."""
    ss = np.random.SeedSequence(w.seed, spawn_key=(99,))
    idx = np.random.Generator(np.random.PCG64(ss)).integers(0, 3, size=w.H)
    return np.array([STA_CANDIDATES[i] for i in idx], dtype=np.int32)


def make_inputs(w: Workload):
    """Return dict with bf16 bits q, k, v [B, L, H, D] (uint16) and windows."""
    shape = (w.B, w.L, w.H, w.D)
    q = _normal(shape, w.seed, 0)
    k = _normal(shape, w.seed, 1)
    v = _normal(shape, w.seed, 2)
    if w.structure == "lowrank":
        _add_lowrank(w, q, k)
    elif w.structure == "smooth":
        _add_smooth(w, q, k)
    elif w.structure != "none":
        raise ValueError(f"unknown structure {w.structure!r}")
    out = {"q": bf16_bits(q), "k": bf16_bits(k), "v": bf16_bits(v)}
    del q, k, v
    if w.mode == "sta":
        out["windows"] = sta_windows(w)
    return out
