"""Block-sparse tiled video attention for MI355X (gfx950).

Python face of libbsta.so.  The four calls of the path keep the C names:

    attn_tile(g, x)                      raster [B,L,H,D] -> tiles [B,Lpad,H,D]
    attn_tile_pool(g, x, pooled=...)     the same, also writing the per-tile means
    attn_select_blocks(g, qt, kt, ...)   pooled scores -> top-k / window -> CSR
    attn_block_sparse_fwd(g, qt, kt, vt, row_ptr, col_idx)   (raster=True: raster output)
    attn_untile(g, yt)                   tiles -> raster

``g`` is a ``Geometry``.  Tensors are torch bfloat16 tensors on the ROCm
device; outputs are allocated with torch when not given.  Every kernel runs on
torch's current stream.  Nothing here computes: each call checks shapes,
marshals pointers and forwards to the C ABI.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
from typing import Optional, Sequence

from . import _lib
from ._lib import SELECT_CUMULATIVE, SELECT_PREPOOLED, SELECT_STA, SELECT_TOPK, BstaError

__all__ = [
    "Geometry", "BstaError", "SELECT_TOPK", "SELECT_STA", "SELECT_CUMULATIVE", "SELECT_PREPOOLED",
    "attn_select_cumulative", "attn_block_sparse_bwd", "attn_block_sparse_bwd_noalloc",
    "attn_prune_queries", "attn_packed_info", "attn_packed_capacity", "attn_select_packed",
    "block_sparse_attention_trainable",
    "attn_tile",
    "attn_tile_pool", "attn_pool", "attn_untile", "attn_select_alloc",
    "attn_select_blocks", "attn_block_sparse_fwd", "attn_geometry", "attn_select_capacity",
    "attn_workspace_bytes", "attn_set_deterministic", "attn_set_key_walk", "WALK_AUTO",
    "WALK_CSR", "WALK_ROTATED", "block_sparse_attention",
]


@dataclasses.dataclass(frozen=True)
class Geometry:
    """Batch, heads, head dim and the (T, Y, X) latent grid.  ``tile_x`` is
    the tile's extent along X: 4 (4x4x4 = 64-token tiles, the default) or 8
    (4x4x8 = 128-token tiles).  A packed sequence (``Geometry.packed``) holds
    ``segments`` instead of a grid: ints are dense segments (rows), 3-tuples
    video regions (latent t, h, w, divided by ``patch``)."""
    B: int
    H: int
    D: int
    T: int
    Y: int
    X: int
    tile_x: int = 4
    segments: Optional[tuple] = None
    patch: tuple = (1, 1, 1)

    @classmethod
    def packed(cls, B, H, D, segments, patch=(1, 1, 1)) -> "Geometry":
        segs = tuple(tuple(int(v) for v in s) if isinstance(s, (tuple, list)) else int(s)
                     for s in segments)
        return cls(B, H, D, 0, 0, 0, 4, segs, tuple(int(p) for p in patch))

    @property
    def c(self) -> _lib.Geom:
        return _lib.geom(self.B, self.H, self.D, self.T, self.Y, self.X, self.tile_x,
                         self.segments, self.patch)

    @property
    def L(self) -> int:
        if self.segments is not None:
            return attn_packed_info(self)["L"]
        return self.T * self.Y * self.X

    @property
    def num_tiles(self) -> int:
        return attn_geometry(self)[0]

    @property
    def Lpad(self) -> int:
        return attn_geometry(self)[1]


def _torch():
    import torch
    return torch


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _expect(t, shape, dtype, name):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on the GPU, got "
                         f"{t.dtype} {tuple(t.shape)} (contiguous={t.is_contiguous()}, "
                         f"device={t.device})")


def attn_geometry(g: Geometry, with_occupancy: bool = False):
    """(Nt, Lpad[, occupancy list]) computed by the library on the host."""
    lib = _lib.load()
    nt = ctypes.c_int32()
    lpad = ctypes.c_int64()
    _lib.check(lib.attn_geometry(ctypes.byref(g.c), ctypes.byref(nt), ctypes.byref(lpad), None))
    if not with_occupancy:
        return nt.value, lpad.value
    occ = (ctypes.c_int32 * nt.value)()
    _lib.check(lib.attn_geometry(ctypes.byref(g.c), None, None, occ))
    return nt.value, lpad.value, list(occ)


def _windows_arg(windows):
    if windows is None:
        return None, None
    flat = [int(v) for row in windows for v in row]
    arr = (ctypes.c_int32 * len(flat))(*flat)
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def attn_select_capacity(g: Geometry, mode: int, topk: int = 0, windows=None) -> int:
    lib = _lib.load()
    _keep, w = _windows_arg(windows)
    return _lib.check(lib.attn_select_capacity(ctypes.byref(g.c), mode, topk, w))


def attn_workspace_bytes(g: Geometry, mode: int) -> int:
    return _lib.check(_lib.load().attn_workspace_bytes(ctypes.byref(g.c), mode))


def attn_tile(g: Geometry, x, out=None):
    torch = _torch()
    _expect(x, (g.B, g.L, g.H, g.D), torch.bfloat16, "x")
    lpad = attn_geometry(g)[1]
    if out is None:
        out = torch.empty((g.B, lpad, g.H, g.D), dtype=torch.bfloat16, device=x.device)
    _expect(out, (g.B, lpad, g.H, g.D), torch.bfloat16, "x_tiled")
    _lib.check(_lib.load().attn_tile(ctypes.byref(g.c), _ptr(x), _ptr(out), _stream()))
    return out


def attn_tile_pool(g: Geometry, x, pooled, out=None):
    """attn_tile plus the per-tile means of the valid rows (fp32 [B, H, Nt, D])
    written to ``pooled`` in the same pass; returns the tiled tensor."""
    torch = _torch()
    _expect(x, (g.B, g.L, g.H, g.D), torch.bfloat16, "x")
    nt, lpad = attn_geometry(g)
    if out is None:
        out = torch.empty((g.B, lpad, g.H, g.D), dtype=torch.bfloat16, device=x.device)
    _expect(out, (g.B, lpad, g.H, g.D), torch.bfloat16, "x_tiled")
    _expect(pooled, (g.B, g.H, nt, g.D), torch.float32, "pooled")
    _lib.check(_lib.load().attn_tile_pool(ctypes.byref(g.c), _ptr(x), _ptr(out), _ptr(pooled),
                                          _stream()))
    return out


def attn_pool(g: Geometry, x_tiled, out=None):
    """Per-tile mean of the valid rows of a tiled tensor: fp32 [B, H, Nt, D]
    (the same vectors attn_tile_pool writes, bit for bit)."""
    torch = _torch()
    nt, lpad = attn_geometry(g)
    _expect(x_tiled, (g.B, lpad, g.H, g.D), torch.bfloat16, "x_tiled")
    if out is None:
        out = torch.empty((g.B, g.H, nt, g.D), dtype=torch.float32, device=x_tiled.device)
    _expect(out, (g.B, g.H, nt, g.D), torch.float32, "pooled")
    _lib.check(_lib.load().attn_pool(ctypes.byref(g.c), _ptr(x_tiled), _ptr(out), _stream()))
    return out


def attn_untile(g: Geometry, y_tiled, out=None):
    torch = _torch()
    lpad = attn_geometry(g)[1]
    _expect(y_tiled, (g.B, lpad, g.H, g.D), torch.bfloat16, "y_tiled")
    if out is None:
        out = torch.empty((g.B, g.L, g.H, g.D), dtype=torch.bfloat16, device=y_tiled.device)
    _expect(out, (g.B, g.L, g.H, g.D), torch.bfloat16, "y")
    _lib.check(_lib.load().attn_untile(ctypes.byref(g.c), _ptr(y_tiled), _ptr(out), _stream()))
    return out


@dataclasses.dataclass
class Selection:
    row_ptr: object        # int32 [B*H*Nt + 1]
    col_idx: object        # int32 [nnz]
    block_mask: object     # uint8 [B, H, Nt, Nt] or None
    workspace: object      # fp32 workspace (pooled Q, K, scores) or None

    def pooled(self, g: Geometry):
        """Views of the pooled Q and K (fp32 [B, H, Nt, D]) left in the workspace."""
        nt = attn_geometry(g)[0]
        n = g.B * g.H * nt * g.D
        ws = self.workspace
        return ws[:n].view(g.B, g.H, nt, g.D), ws[n:2 * n].view(g.B, g.H, nt, g.D)

    def scores(self, g: Geometry):
        nt = attn_geometry(g)[0]
        n = g.B * g.H * nt * g.D
        return self.workspace[2 * n:2 * n + g.B * g.H * nt * nt].view(g.B, g.H, nt, nt)


def attn_select_alloc(g: Geometry, mode: int = SELECT_TOPK, topk: int = 0, windows=None,
                      want_mask: bool = True, device="cuda") -> Selection:
    """Output buffers and workspace for attn_select_blocks.  With the top-k
    mode, ``Selection.pooled(g)`` views are where attn_tile_pool writes."""
    torch = _torch()
    nt = attn_geometry(g)[0]
    cap = attn_select_capacity(g, mode, topk, windows)
    wsb = attn_workspace_bytes(g, mode)
    return Selection(
        row_ptr=torch.empty(g.B * g.H * nt + 1, dtype=torch.int32, device=device),
        col_idx=torch.empty(max(cap, 1), dtype=torch.int32, device=device),
        block_mask=(torch.empty((g.B, g.H, nt, nt), dtype=torch.uint8, device=device)
                    if want_mask else None),
        workspace=(torch.empty(wsb // 4, dtype=torch.float32, device=device) if wsb > 0 else None))


def _check_selection(g: Geometry, sel: Selection):
    """Shapes and dtypes of a caller-supplied Selection against the geometry
    (the C ABI sees only pointers and the col_idx / workspace sizes)."""
    torch = _torch()
    nt = attn_geometry(g)[0]
    _expect(sel.row_ptr, (g.B * g.H * nt + 1,), torch.int32, "out.row_ptr")
    _expect(sel.block_mask, (g.B, g.H, nt, nt), torch.uint8, "out.block_mask")
    for name, t, dt in (("out.col_idx", sel.col_idx, torch.int32),
                        ("out.workspace", sel.workspace, torch.float32)):
        if t is not None and (t.dtype != dt or t.dim() != 1 or not t.is_contiguous() or not t.is_cuda):
            raise ValueError(f"{name}: expected a contiguous 1-D {dt} tensor on the GPU, got "
                             f"{t.dtype} {tuple(t.shape)}")


def attn_select_blocks(g: Geometry, q_tiled, k_tiled, mode: int = SELECT_TOPK, topk: int = 0,
                       windows: Optional[Sequence[Sequence[int]]] = None, want_mask: bool = True,
                       out: Optional[Selection] = None) -> Selection:
    """Coarse stage.  ``mode`` may be SELECT_TOPK | SELECT_PREPOOLED when
    ``out`` (from attn_select_alloc) already holds the pooled Q and K written
    by attn_tile_pool; q_tiled and k_tiled are then not read (may be None)."""
    torch = _torch()
    nt, lpad = attn_geometry(g)
    prepooled = bool(mode & SELECT_PREPOOLED)
    if mode == SELECT_TOPK:
        _expect(q_tiled, (g.B, lpad, g.H, g.D), torch.bfloat16, "q_tiled")
        _expect(k_tiled, (g.B, lpad, g.H, g.D), torch.bfloat16, "k_tiled")
    if prepooled and (out is None or out.workspace is None):
        raise ValueError("SELECT_PREPOOLED needs `out` holding the pooled Q and K")
    if out is None:
        dev = (q_tiled if q_tiled is not None else torch.empty(0, device="cuda")).device
        out = attn_select_alloc(g, mode, topk, windows, want_mask, dev)
    _check_selection(g, out)
    _keep, w = _windows_arg(windows)
    ws = out.workspace
    status = _lib.load().attn_select_blocks(
        ctypes.byref(g.c), _ptr(q_tiled), _ptr(k_tiled), mode, topk, w, _ptr(out.block_mask),
        _ptr(out.row_ptr), _ptr(out.col_idx), out.col_idx.numel(), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream())
    _lib.check(status)
    return out


def attn_select_cumulative(g: Geometry, q_tiled, k_tiled, threshold: float, min_blocks: int = 0,
                           prepooled: bool = False, want_mask: bool = True,
                           out: Optional[Selection] = None) -> Selection:
    """Coarse stage with a cumulative probability threshold: each query tile
    keeps the shortest run of its best key tiles whose softmax(S/sqrt(D))
    mass reaches ``threshold`` (and at least ``min_blocks``).  Row lengths
    vary: ``row_ptr[-1]`` is the entry count, and ``col_idx`` is sized for
    the worst case.  With ``prepooled``, ``out`` (from attn_select_alloc with
    SELECT_CUMULATIVE) already holds the pooled Q and K from attn_tile_pool."""
    torch = _torch()
    nt, lpad = attn_geometry(g)
    if not prepooled:
        _expect(q_tiled, (g.B, lpad, g.H, g.D), torch.bfloat16, "q_tiled")
        _expect(k_tiled, (g.B, lpad, g.H, g.D), torch.bfloat16, "k_tiled")
    elif out is None or out.workspace is None:
        raise ValueError("prepooled needs `out` holding the pooled Q and K")
    if out is None:
        out = attn_select_alloc(g, SELECT_CUMULATIVE, 0, None, want_mask, q_tiled.device)
    _check_selection(g, out)
    ws = out.workspace
    status = _lib.load().attn_select_cumulative(
        ctypes.byref(g.c), _ptr(q_tiled), _ptr(k_tiled), SELECT_PREPOOLED if prepooled else 0,
        float(threshold), int(min_blocks), _ptr(out.block_mask), _ptr(out.row_ptr),
        _ptr(out.col_idx), out.col_idx.numel(), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream())
    _lib.check(status)
    return out


def attn_packed_info(g: Geometry) -> dict:
    """Layout of a packed geometry, from the library: ``num_prefix`` (tiles
    of the dense segments), ``spans`` (tile range of each video region) and
    ``L`` (packed length)."""
    lib = _lib.load()
    c = g.c
    npre, nreg, plen = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    _lib.check(lib.attn_packed_info(ctypes.byref(c), ctypes.byref(npre), ctypes.byref(nreg), None,
                                    ctypes.byref(plen)))
    spans = (ctypes.c_int32 * (2 * nreg.value))()
    _lib.check(lib.attn_packed_info(ctypes.byref(c), None, None, spans, None))
    return {"num_prefix": npre.value, "L": plen.value,
            "spans": [(spans[2 * r], spans[2 * r + 1]) for r in range(nreg.value)]}


def attn_packed_capacity(g: Geometry, sparsity: float, ref_keep_rate: Optional[float] = None,
                         exempt: bool = True) -> int:
    rk = float("nan") if ref_keep_rate is None else float(ref_keep_rate)
    return _lib.check(_lib.load().attn_packed_capacity(ctypes.byref(g.c), float(sparsity), rk,
                                                       int(bool(exempt))))


def attn_select_packed(g: Geometry, q_tiled, k_tiled, sparsity: float,
                       ref_keep_rate: Optional[float] = None, exempt: bool = True,
                       prepooled: bool = False, want_mask: bool = True,
                       out: Optional[Selection] = None) -> Selection:
    """Coarse stage of a packed sequence.  Exempt mode: prefix query tiles
    keep every tile; video query tiles keep the prefix and, per video region,
    its k best tiles (reference regions at ``ref_keep_rate``, the last region
    at 1 - ``sparsity``).  Compete mode (one region): the k best tiles of the
    whole sequence.  ``prepooled``: ``out`` (from attn_select_alloc with
    SELECT_TOPK) already holds the pooled Q and K from attn_tile_pool."""
    torch = _torch()
    nt, lpad = attn_geometry(g)
    if not prepooled:
        _expect(q_tiled, (g.B, lpad, g.H, g.D), torch.bfloat16, "q_tiled")
        _expect(k_tiled, (g.B, lpad, g.H, g.D), torch.bfloat16, "k_tiled")
    elif out is None or out.workspace is None:
        raise ValueError("prepooled needs `out` holding the pooled Q and K")
    cap = attn_packed_capacity(g, sparsity, ref_keep_rate, exempt)
    if out is None:
        wsb = attn_workspace_bytes(g, SELECT_TOPK)
        dev = q_tiled.device
        out = Selection(
            row_ptr=torch.empty(g.B * g.H * nt + 1, dtype=torch.int32, device=dev),
            col_idx=torch.empty(max(cap, 1), dtype=torch.int32, device=dev),
            block_mask=(torch.empty((g.B, g.H, nt, nt), dtype=torch.uint8, device=dev)
                        if want_mask else None),
            workspace=torch.empty(wsb // 4, dtype=torch.float32, device=dev))
    _check_selection(g, out)
    ws = out.workspace
    rk = float("nan") if ref_keep_rate is None else float(ref_keep_rate)
    status = _lib.load().attn_select_packed(
        ctypes.byref(g.c), _ptr(q_tiled), _ptr(k_tiled), SELECT_PREPOOLED if prepooled else 0,
        float(sparsity), rk, int(bool(exempt)), _ptr(out.block_mask), _ptr(out.row_ptr),
        _ptr(out.col_idx), out.col_idx.numel(), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream())
    _lib.check(status)
    return out


def attn_prune_queries(g: Geometry, q_tiled, keep_ratio: float, pooled=None, keep_mask=None,
                       keep_count=None):
    """Query pruning: each tile keeps min(n, max(1, floor(keep_ratio * n))) of
    its n valid query tokens, those least aligned with the tile's mean query.
    Returns (keep_mask, keep_count, pooled): keep_mask int64 [B, H, Nt * U]
    holding a 64-bit kept-slot mask per 64-slot unit (U = tile_x // 4 units
    per tile; word u of tile j covers its slots 64u + [0, 64), bit r = slot
    64u + r), keep_count int32 [B, H, Nt], pooled fp32 [B, H, Nt, D] the kept
    queries' means.  Give ``pooled`` = Selection.pooled(g)[0] to select key
    tiles from them."""
    torch = _torch()
    nt, lpad = attn_geometry(g)
    nu = nt * (g.tile_x // 4)
    _expect(q_tiled, (g.B, lpad, g.H, g.D), torch.bfloat16, "q_tiled")
    dev = q_tiled.device
    if keep_mask is None:
        keep_mask = torch.empty((g.B, g.H, nu), dtype=torch.int64, device=dev)
    if keep_count is None:
        keep_count = torch.empty((g.B, g.H, nt), dtype=torch.int32, device=dev)
    if pooled is None:
        pooled = torch.empty((g.B, g.H, nt, g.D), dtype=torch.float32, device=dev)
    _expect(keep_mask, (g.B, g.H, nu), torch.int64, "keep_mask")
    _expect(keep_count, (g.B, g.H, nt), torch.int32, "keep_count")
    _expect(pooled, (g.B, g.H, nt, g.D), torch.float32, "pooled")
    _lib.check(_lib.load().attn_prune_queries(ctypes.byref(g.c), _ptr(q_tiled), float(keep_ratio),
                                              _ptr(keep_mask), _ptr(keep_count), _ptr(pooled),
                                              _stream()))
    return keep_mask, keep_count, pooled


def attn_block_sparse_fwd(g: Geometry, q_tiled, k_tiled, v_tiled, row_ptr, col_idx,
                          softmax_scale: Optional[float] = None, causal: bool = False,
                          out=None, lse=None, want_lse: bool = False, raster: bool = False,
                          keep=None):
    """Block-sparse attention over the tiled tensors.  The output is tiled
    [B, Lpad, H, D], or with ``raster=True`` written straight to raster order
    [B, L, H, D] (attn_block_sparse_fwd_raster: no separate untile pass).
    ``keep`` (the keep_mask of attn_prune_queries) restricts the output rows
    to the kept query slots (attn_block_sparse_fwd_pruned); the others are
    written as zeros."""
    torch = _torch()
    nt, lpad = attn_geometry(g)
    for name, t in (("q_tiled", q_tiled), ("k_tiled", k_tiled), ("v_tiled", v_tiled)):
        _expect(t, (g.B, lpad, g.H, g.D), torch.bfloat16, name)
    _expect(row_ptr, (g.B * g.H * nt + 1,), torch.int32, "row_ptr")
    if col_idx.dtype != torch.int32 or not col_idx.is_contiguous():
        raise ValueError("col_idx: expected contiguous int32")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(g.D)
    rows = g.L if raster else lpad
    if out is None:
        out = torch.empty((g.B, rows, g.H, g.D), dtype=torch.bfloat16, device=q_tiled.device)
    _expect(out, (g.B, rows, g.H, g.D), torch.bfloat16, "o" if raster else "o_tiled")
    if lse is None and want_lse:
        lse = torch.empty((g.B, g.H, lpad), dtype=torch.float32, device=q_tiled.device)
    _expect(lse, (g.B, g.H, lpad), torch.float32, "lse")
    lib = _lib.load()
    if keep is not None:
        _expect(keep, (g.B, g.H, nt * (g.tile_x // 4)), torch.int64, "keep")
        _lib.check(lib.attn_block_sparse_fwd_pruned(
            ctypes.byref(g.c), _ptr(q_tiled), _ptr(k_tiled), _ptr(v_tiled), _ptr(row_ptr),
            _ptr(col_idx), col_idx.numel(), float(softmax_scale), int(bool(causal)), _ptr(keep),
            int(bool(raster)), _ptr(out), _ptr(lse), _stream()))
        return (out, lse) if want_lse or lse is not None else out
    fn = lib.attn_block_sparse_fwd_raster if raster else lib.attn_block_sparse_fwd
    _lib.check(fn(
        ctypes.byref(g.c), _ptr(q_tiled), _ptr(k_tiled), _ptr(v_tiled), _ptr(row_ptr),
        _ptr(col_idx), col_idx.numel(), float(softmax_scale), int(bool(causal)), _ptr(out),
        _ptr(lse), _stream()))
    return (out, lse) if want_lse or lse is not None else out


def attn_block_sparse_bwd(g: Geometry, q_tiled, k_tiled, v_tiled, o_tiled, do_tiled, lse, row_ptr,
                          col_idx, softmax_scale: Optional[float] = None, out=None):
    """Gradients (dq, dk, dv), tiled bf16 [B, Lpad, H, D], of sum(do * o) for
    o = attn_block_sparse_fwd(...) (tiled output) with its lse.  ``out`` may
    give the three output tensors."""
    torch = _torch()
    nt, lpad = attn_geometry(g)
    for name, t in (("q_tiled", q_tiled), ("k_tiled", k_tiled), ("v_tiled", v_tiled),
                    ("o_tiled", o_tiled), ("do_tiled", do_tiled)):
        _expect(t, (g.B, lpad, g.H, g.D), torch.bfloat16, name)
    _expect(lse, (g.B, g.H, lpad), torch.float32, "lse")
    _expect(row_ptr, (g.B * g.H * nt + 1,), torch.int32, "row_ptr")
    if col_idx.dtype != torch.int32 or not col_idx.is_contiguous():
        raise ValueError("col_idx: expected contiguous int32")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(g.D)
    if out is None:
        out = tuple(torch.empty_like(q_tiled) for _ in range(3))
    for name, t in zip(("dq", "dk", "dv"), out):
        _expect(t, (g.B, lpad, g.H, g.D), torch.bfloat16, name)
    lib = _lib.load()
    wsb = lib.attn_bwd_workspace_bytes(ctypes.byref(g.c), col_idx.numel())
    _lib.check(wsb)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=q_tiled.device)
    _lib.check(lib.attn_block_sparse_bwd(
        ctypes.byref(g.c), _ptr(q_tiled), _ptr(k_tiled), _ptr(v_tiled), _ptr(o_tiled),
        _ptr(do_tiled), _ptr(lse), _ptr(row_ptr), _ptr(col_idx), col_idx.numel(),
        float(softmax_scale), 0, _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _ptr(ws), wsb,
        _stream()))
    return out


def attn_block_sparse_bwd_noalloc(g: Geometry, q_tiled, k_tiled, v_tiled, o_tiled, do_tiled, lse,
                                  row_ptr, col_idx, out, softmax_scale: Optional[float] = None):
    """attn_block_sparse_bwd with the library's static 64 MiB device scratch
    as its workspace: allocates nothing (the caller gives ``out`` = (dq, dk,
    dv)).  Equal to attn_block_sparse_bwd bit for bit; raises BstaError
    (capacity) when the workspace it needs exceeds the scratch.  Calls that
    overlap on one GPU share the scratch and race."""
    torch = _torch()
    nt, lpad = attn_geometry(g)
    for name, t in (("q_tiled", q_tiled), ("k_tiled", k_tiled), ("v_tiled", v_tiled),
                    ("o_tiled", o_tiled), ("do_tiled", do_tiled)):
        _expect(t, (g.B, lpad, g.H, g.D), torch.bfloat16, name)
    _expect(lse, (g.B, g.H, lpad), torch.float32, "lse")
    _expect(row_ptr, (g.B * g.H * nt + 1,), torch.int32, "row_ptr")
    if col_idx.dtype != torch.int32 or not col_idx.is_contiguous():
        raise ValueError("col_idx: expected contiguous int32")
    if out is None or len(out) != 3:
        raise ValueError("out: give the three output tensors (dq, dk, dv)")
    for name, t in zip(("dq", "dk", "dv"), out):
        _expect(t, (g.B, lpad, g.H, g.D), torch.bfloat16, name)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(g.D)
    _lib.check(_lib.load().attn_block_sparse_bwd_noalloc(
        ctypes.byref(g.c), _ptr(q_tiled), _ptr(k_tiled), _ptr(v_tiled), _ptr(o_tiled),
        _ptr(do_tiled), _ptr(lse), _ptr(row_ptr), _ptr(col_idx), col_idx.numel(),
        float(softmax_scale), 0, _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _stream()))
    return out


# Key walks of attn_block_sparse_fwd (attn_set_key_walk).
WALK_AUTO, WALK_CSR, WALK_ROTATED = 0, 1, 2


def attn_set_key_walk(mode: int) -> int:
    """Process-wide key order of attn_block_sparse_fwd: WALK_AUTO (the
    default: the cache-friendly rotated walk for large heads whose rows
    spread over the key range, CSR order otherwise), WALK_CSR (every row in
    CSR order, bitwise reproducible) or WALK_ROTATED (every row rotated).
    Returns the previous mode."""
    if mode not in (WALK_AUTO, WALK_CSR, WALK_ROTATED):
        raise ValueError(f"key walk {mode!r}: WALK_AUTO, WALK_CSR or WALK_ROTATED")
    return int(_lib.load().attn_set_deterministic(int(mode)))


def attn_set_deterministic(enable: bool) -> bool:
    """True: every CSR row walked in order (WALK_CSR, bitwise reproducible);
    False: the default walk (WALK_AUTO).  Returns whether the previous mode
    was WALK_CSR."""
    return attn_set_key_walk(WALK_CSR if enable else WALK_AUTO) == WALK_CSR


def block_sparse_attention(g: Geometry, q, k, v, mode: int = SELECT_TOPK, topk: int = 0,
                           windows=None, threshold: Optional[float] = None, min_blocks: int = 0,
                           query_keep_ratio: Optional[float] = None):
    """The whole path on raster [B, L, H, D] tensors: tile, select, attend, untile.
    ``mode`` is SELECT_TOPK (``topk``), SELECT_STA (``windows``) or
    SELECT_CUMULATIVE (``threshold``, ``min_blocks``).  With top-k and the
    cumulative threshold Q and K are pooled while they are tiled; the
    attention writes its output in raster order directly.  With
    ``query_keep_ratio`` (top-k or cumulative) the queries are pruned first
    (attn_prune_queries): key tiles are selected from the kept queries'
    means and pruned query rows come out as zeros."""
    keep = None
    if mode in (SELECT_TOPK, SELECT_CUMULATIVE):
        sel = attn_select_alloc(g, mode, topk, want_mask=False, device=q.device)
        pq, pk = sel.pooled(g)
        if query_keep_ratio is None:
            qt = attn_tile_pool(g, q, pq)
        else:
            qt = attn_tile(g, q)
            keep, _, _ = attn_prune_queries(g, qt, query_keep_ratio, pooled=pq)
        kt = attn_tile_pool(g, k, pk)
        vt = attn_tile(g, v)
        if mode == SELECT_TOPK:
            sel = attn_select_blocks(g, None, None, SELECT_TOPK | SELECT_PREPOOLED, topk, out=sel)
        else:
            if threshold is None:
                raise ValueError("SELECT_CUMULATIVE needs a threshold")
            sel = attn_select_cumulative(g, None, None, threshold, min_blocks, prepooled=True,
                                         out=sel)
    else:
        if query_keep_ratio is not None:
            raise ValueError("query pruning selects from the kept queries: use SELECT_TOPK or "
                             "SELECT_CUMULATIVE")
        qt, kt, vt = attn_tile(g, q), attn_tile(g, k), attn_tile(g, v)
        sel = attn_select_blocks(g, qt, kt, mode, topk, windows, want_mask=False)
    return attn_block_sparse_fwd(g, qt, kt, vt, sel.row_ptr, sel.col_idx, raster=True, keep=keep)


def _select_for(g: Geometry, qt, kt, mode, topk, windows, threshold, min_blocks):
    if mode == SELECT_CUMULATIVE:
        if threshold is None:
            raise ValueError("SELECT_CUMULATIVE needs a threshold")
        return attn_select_cumulative(g, qt, kt, threshold, min_blocks, want_mask=False)
    return attn_select_blocks(g, qt, kt, mode, topk, windows, want_mask=False)


def block_sparse_attention_trainable(g: Geometry, q, k, v, mode: int = SELECT_TOPK, topk: int = 0,
                                     windows=None, threshold: Optional[float] = None,
                                     min_blocks: int = 0):
    """The whole path as a differentiable torch op on raster [B, L, H, D]
    tensors: the forward tiles, selects and attends (keeping the tiled
    output and lse), and backward() runs attn_block_sparse_bwd on the tiled
    gradient and untiles dq, dk, dv.  The block selection is discrete and
    passes no gradient."""
    torch = _torch()

    class _Fn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q_, k_, v_):
            qt, kt, vt = attn_tile(g, q_), attn_tile(g, k_), attn_tile(g, v_)
            sel = _select_for(g, qt, kt, mode, topk, windows, threshold, min_blocks)
            ot, lse = attn_block_sparse_fwd(g, qt, kt, vt, sel.row_ptr, sel.col_idx,
                                            want_lse=True)
            ctx.save_for_backward(qt, kt, vt, ot, lse, sel.row_ptr, sel.col_idx)
            return attn_untile(g, ot)

        @staticmethod
        def backward(ctx, do):
            qt, kt, vt, ot, lse, rp, ci = ctx.saved_tensors
            dot = attn_tile(g, do.contiguous())
            dq, dk, dv = attn_block_sparse_bwd(g, qt, kt, vt, ot, dot, lse, rp, ci)
            return attn_untile(g, dq), attn_untile(g, dk), attn_untile(g, dv)

    return _Fn.apply(q, k, v)
