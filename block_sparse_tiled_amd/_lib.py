"""ctypes binding of libbsta.so (argument marshalling only).

Every function here forwards to the C ABI declared in include/bsta.h with
the same name.  Tensors are torch tensors on a ROCm device; only their data
pointers, the geometry and the current HIP stream cross the boundary.  A
non-zero status raises BstaError carrying attn_last_error().  There is no
fallback: if the library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbsta.so")

BSTA_OK = 0
BSTA_ERR_NULL = -1
BSTA_ERR_SHAPE = -2
BSTA_ERR_UNSUPPORTED = -3
BSTA_ERR_CAPACITY = -4
BSTA_ERR_HIP = -5
SELECT_TOPK = 0
SELECT_STA = 1
SELECT_CUMULATIVE = 2
SELECT_PREPOOLED = 0x100
MAX_STA_HEADS = 256

EXPORTS = (
    "attn_geometry", "attn_tile", "attn_tile_pool", "attn_pool", "attn_untile", "attn_select_capacity",
    "attn_workspace_bytes", "attn_select_blocks", "attn_select_cumulative",
    "attn_block_sparse_fwd",
    "attn_block_sparse_fwd_raster", "attn_bwd_workspace_bytes", "attn_block_sparse_bwd",
    "attn_block_sparse_bwd_noalloc", "attn_prune_queries", "attn_block_sparse_fwd_pruned",
    "attn_packed_info", "attn_packed_capacity", "attn_select_packed",
    "attn_status_string", "attn_last_error", "attn_set_deterministic",
)


class BstaError(ValueError):
    """A libbsta call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


MAX_SEGMENTS = 16


class Segments(ctypes.Structure):
    """bsta_segments: a packed sequence of dense segments and video regions."""
    _fields_ = [("count", ctypes.c_int32), ("patch", ctypes.c_int32 * 3),
                ("kind", ctypes.c_int32 * MAX_SEGMENTS), ("rows", ctypes.c_int32 * MAX_SEGMENTS),
                ("shape", (ctypes.c_int32 * 3) * MAX_SEGMENTS)]


class Geom(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "H", "D", "T", "Y", "X", "tile_t", "tile_y", "tile_x")] + [
                    ("segments", ctypes.POINTER(Segments))]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libbsta.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    G = ctypes.POINTER(Geom)
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    sig = {
        "attn_geometry": (i32, [G, ctypes.POINTER(i32), ctypes.POINTER(i64), P]),
        "attn_tile": (i32, [G, P, P, P]),
        "attn_tile_pool": (i32, [G, P, P, P, P]),
        "attn_untile": (i32, [G, P, P, P]),
        "attn_pool": (i32, [G, P, P, P]),
        "attn_select_capacity": (i64, [G, i32, i32, P]),
        "attn_workspace_bytes": (i64, [G, i32]),
        "attn_select_blocks": (i32, [G, P, P, i32, i32, P, P, P, P, i64, P, i64, P]),
        "attn_select_cumulative": (i32, [G, P, P, i32, ctypes.c_float, i32, P, P, P, i64, P, i64, P]),
        "attn_block_sparse_fwd": (i32, [G, P, P, P, P, P, i64, ctypes.c_float, i32, P, P, P]),
        "attn_block_sparse_fwd_raster": (i32, [G, P, P, P, P, P, i64, ctypes.c_float, i32, P, P, P]),
        "attn_bwd_workspace_bytes": (i64, [G, i64]),
        "attn_block_sparse_bwd": (i32, [G, P, P, P, P, P, P, P, P, i64, ctypes.c_float, i32, P, P, P,
                                        P, i64, P]),
        "attn_block_sparse_bwd_noalloc": (i32, [G, P, P, P, P, P, P, P, P, i64, ctypes.c_float, i32,
                                                P, P, P, P]),
        "attn_prune_queries": (i32, [G, P, ctypes.c_double, P, P, P, P]),
        "attn_block_sparse_fwd_pruned": (i32, [G, P, P, P, P, P, i64, ctypes.c_float, i32, P, i32, P,
                                               P, P]),
        "attn_packed_info": (i32, [G, ctypes.POINTER(i32), ctypes.POINTER(i32), P,
                                   ctypes.POINTER(i64)]),
        "attn_packed_capacity": (i64, [G, ctypes.c_double, ctypes.c_double, i32]),
        "attn_select_packed": (i32, [G, P, P, i32, ctypes.c_double, ctypes.c_double, i32, P, P, P,
                                     i64, P, i64, P]),
        "attn_status_string": (ctypes.c_char_p, [i32]),
        "attn_last_error": (ctypes.c_char_p, []),
        "attn_set_deterministic": (i32, [i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(status: int) -> int:
    if status < 0:
        lib = load()
        raise BstaError(int(status), lib.attn_last_error().decode())
    return status


def segments(packed, patch=(1, 1, 1)) -> Segments:
    """bsta_segments of a packed list: ints are dense segments (rows),
    3-tuples video regions (latent t, h, w)."""
    if len(packed) > MAX_SEGMENTS:
        raise ValueError(f"at most {MAX_SEGMENTS} segments, got {len(packed)}")
    sg = Segments()
    sg.count = len(packed)
    for ax in range(3):
        sg.patch[ax] = int(patch[ax])
    for i, seg in enumerate(packed):
        if isinstance(seg, (tuple, list)):
            sg.kind[i] = 1
            for ax in range(3):
                sg.shape[i][ax] = int(seg[ax])
        else:
            sg.rows[i] = int(seg)
    return sg


def geom(B, H, D, T, Y, X, tile_x=4, packed=None, patch=(1, 1, 1)) -> Geom:
    g = Geom(int(B), int(H), int(D), int(T), int(Y), int(X), 4, 4, int(tile_x))
    if packed is not None:
        g.segments = ctypes.pointer(segments(packed, patch))  # kept alive by g
    return g
