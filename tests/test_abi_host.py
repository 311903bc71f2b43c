"""Host-side contract of libbsta.so: exports, geometry, argument checks.

Nothing here launches a kernel: every call either is host-only (geometry,
capacity, workspace size) or fails its argument checks before any HIP call,
so the tests run without a GPU.  Pointers passed to failing calls are dummies
that the library never dereferences.
"""
import ctypes
import math
import os
import re
import subprocess

import numpy as np
import pytest

from block_sparse_tiled_amd import _lib
from oracle import geometry

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x1000)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libbsta.so not built")
    return _lib.load()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "bsta.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


def test_header_declarations_are_exported(lib):
    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r"\bT (attn_[a-z_]+)$", nm, flags=re.M))
    assert set(declared) <= exported


def _g(B=1, H=2, D=64, T=8, Y=8, X=8, tile=(4, 4, 4)):
    return _lib.Geom(B, H, D, T, Y, X, *tile)


@pytest.mark.parametrize("grid", [(8, 8, 8), (21, 30, 52), (20, 48, 80), (5, 6, 7), (1, 1, 1)])
def test_geometry_matches_oracle(lib, grid):
    T, Y, X = grid
    g = _g(T=T, Y=Y, X=X)
    nt, lpad = ctypes.c_int32(), ctypes.c_int64()
    assert lib.attn_geometry(ctypes.byref(g), ctypes.byref(nt), ctypes.byref(lpad), None) == 0
    assert nt.value == geometry.num_tiles(T, Y, X)
    assert lpad.value == geometry.padded_len(T, Y, X)
    occ = (ctypes.c_int32 * nt.value)()
    assert lib.attn_geometry(ctypes.byref(g), None, None, occ) == 0
    assert np.array_equal(np.array(occ), geometry.occupancy(T, Y, X))


def test_capacity_and_workspace(lib):
    g = _g(B=2, H=3, D=128, T=16, Y=48, X=80)
    nt = geometry.num_tiles(16, 48, 80)
    assert lib.attn_select_capacity(ctypes.byref(g), 0, 7, None) == 2 * 3 * nt * 7
    win = (ctypes.c_int32 * 9)(1, 3, 3, 3, 3, 3, 3, 5, 5)
    assert lib.attn_select_capacity(ctypes.byref(g), 1, 0, win) == 2 * nt * (9 + 27 + 75)
    assert lib.attn_workspace_bytes(ctypes.byref(g), 0) == 4 * (2 * 2 * 3 * nt * 128 + 2 * 3 * nt * nt)
    assert lib.attn_workspace_bytes(ctypes.byref(g), 1) == 0
    # The prepooled flag changes neither the CSR size nor the workspace (it
    # only says the workspace already holds pooled Q and K) ...
    pre = _lib.SELECT_TOPK | _lib.SELECT_PREPOOLED
    assert lib.attn_select_capacity(ctypes.byref(g), pre, 7, None) == 2 * 3 * nt * 7
    assert lib.attn_workspace_bytes(ctypes.byref(g), pre) == lib.attn_workspace_bytes(ctypes.byref(g), 0)
    # ... and applies to top-k only.
    sta_pre = _lib.SELECT_STA | _lib.SELECT_PREPOOLED
    assert lib.attn_select_capacity(ctypes.byref(g), sta_pre, 0, win) == _lib.BSTA_ERR_UNSUPPORTED
    assert lib.attn_workspace_bytes(ctypes.byref(g), sta_pre) == _lib.BSTA_ERR_UNSUPPORTED


def _err(lib):
    return lib.attn_last_error().decode()


def test_geometry_errors(lib):
    assert lib.attn_geometry(None, None, None, None) == _lib.BSTA_ERR_NULL
    assert lib.attn_geometry(ctypes.byref(_g(D=96)), None, None, None) == _lib.BSTA_ERR_UNSUPPORTED
    assert "D=96" in _err(lib)
    assert lib.attn_geometry(ctypes.byref(_g(tile=(8, 8, 8))), None, None, None) == _lib.BSTA_ERR_UNSUPPORTED
    assert lib.attn_geometry(ctypes.byref(_g(B=0)), None, None, None) == _lib.BSTA_ERR_SHAPE
    assert lib.attn_geometry(ctypes.byref(_g(T=0)), None, None, None) == _lib.BSTA_ERR_SHAPE
    assert lib.attn_geometry(ctypes.byref(_g(X=-3)), None, None, None) == _lib.BSTA_ERR_SHAPE


def test_tile_errors(lib):
    assert lib.attn_tile(ctypes.byref(_g()), None, FAKE, None) == _lib.BSTA_ERR_NULL
    assert lib.attn_tile(ctypes.byref(_g()), FAKE, None, None) == _lib.BSTA_ERR_NULL
    assert lib.attn_untile(ctypes.byref(_g()), None, FAKE, None) == _lib.BSTA_ERR_NULL
    assert lib.attn_tile(ctypes.byref(_g(D=32)), FAKE, FAKE, None) == _lib.BSTA_ERR_UNSUPPORTED
    for x, xt, pooled in ((None, FAKE, FAKE), (FAKE, None, FAKE), (FAKE, FAKE, None)):
        assert lib.attn_tile_pool(ctypes.byref(_g()), x, xt, pooled, None) == _lib.BSTA_ERR_NULL
    assert lib.attn_tile_pool(ctypes.byref(_g(D=32)), FAKE, FAKE, FAKE, None) == _lib.BSTA_ERR_UNSUPPORTED


def _select(lib, g, mode=0, topk=2, win=None, rp=FAKE, ci=FAKE, cap=10 ** 9, ws=FAKE, wsb=10 ** 12,
            q=FAKE, k=FAKE):
    return lib.attn_select_blocks(ctypes.byref(g), q, k, mode, topk, win, None, rp, ci, cap, ws,
                                  wsb, None)


def test_select_errors(lib):
    g = _g()  # 8 tiles
    assert _select(lib, g, topk=0) == _lib.BSTA_ERR_SHAPE
    assert _select(lib, g, topk=9) == _lib.BSTA_ERR_SHAPE
    assert "topk=9" in _err(lib)
    assert _select(lib, g, mode=5) == _lib.BSTA_ERR_UNSUPPORTED
    assert _select(lib, g, rp=None) == _lib.BSTA_ERR_NULL
    assert _select(lib, g, ci=None) == _lib.BSTA_ERR_NULL
    assert _select(lib, g, q=None) == _lib.BSTA_ERR_NULL
    assert _select(lib, g, ws=None) == _lib.BSTA_ERR_NULL
    pre = _lib.SELECT_TOPK | _lib.SELECT_PREPOOLED
    assert _select(lib, g, mode=pre, ws=None, q=None, k=None) == _lib.BSTA_ERR_NULL
    assert "workspace" in _err(lib)
    assert _select(lib, g, mode=_lib.SELECT_STA | _lib.SELECT_PREPOOLED) == _lib.BSTA_ERR_UNSUPPORTED
    need = 1 * 2 * 8 * 2
    assert _select(lib, g, cap=need - 1) == _lib.BSTA_ERR_CAPACITY
    wsb = lib.attn_workspace_bytes(ctypes.byref(g), 0)
    assert _select(lib, g, wsb=wsb - 1) == _lib.BSTA_ERR_CAPACITY
    # window mode
    assert _select(lib, g, mode=1, win=None) == _lib.BSTA_ERR_NULL
    bad = (ctypes.c_int32 * 6)(1, 1, 3, 1, 1, 1)   # 3 > 2 tiles along X
    assert _select(lib, g, mode=1, win=bad) == _lib.BSTA_ERR_SHAPE
    zero = (ctypes.c_int32 * 6)(1, 0, 1, 1, 1, 1)
    assert _select(lib, g, mode=1, win=zero) == _lib.BSTA_ERR_SHAPE
    good = (ctypes.c_int32 * 6)(2, 2, 2, 1, 1, 1)
    assert _select(lib, g, mode=1, win=good, cap=8 * 9 - 1) == _lib.BSTA_ERR_CAPACITY
    many = _g(H=_lib.MAX_STA_HEADS + 1)
    w = (ctypes.c_int32 * (3 * (_lib.MAX_STA_HEADS + 1)))(*([1] * 3 * (_lib.MAX_STA_HEADS + 1)))
    assert _select(lib, many, mode=1, win=w) == _lib.BSTA_ERR_SHAPE


def test_cumulative_capacity_and_workspace(lib):
    g = _g(B=2, H=3, D=128, T=16, Y=48, X=80)
    nt = geometry.num_tiles(16, 48, 80)
    cum = _lib.SELECT_CUMULATIVE
    # Row lengths depend on the data: room for every row to keep all tiles.
    assert lib.attn_select_capacity(ctypes.byref(g), cum, 0, None) == 2 * 3 * nt * nt
    assert lib.attn_workspace_bytes(ctypes.byref(g), cum) == lib.attn_workspace_bytes(ctypes.byref(g), 0)
    pre = cum | _lib.SELECT_PREPOOLED
    assert lib.attn_workspace_bytes(ctypes.byref(g), pre) == lib.attn_workspace_bytes(ctypes.byref(g), 0)


def _cum(lib, g, flags=0, tau=0.5, mb=0, rp=FAKE, ci=FAKE, cap=10 ** 12, ws=FAKE, wsb=10 ** 12,
         q=FAKE, k=FAKE):
    return lib.attn_select_cumulative(ctypes.byref(g), q, k, flags, tau, mb, None, rp, ci, cap, ws,
                                      wsb, None)


def test_cumulative_errors(lib):
    g = _g()  # 8 tiles
    for tau in (0.0, -0.25, 1.5, float("nan")):
        assert _cum(lib, g, tau=tau) == _lib.BSTA_ERR_SHAPE
        assert "threshold" in _err(lib)
    assert _cum(lib, g, mb=-1) == _lib.BSTA_ERR_SHAPE
    assert _cum(lib, g, flags=7) == _lib.BSTA_ERR_UNSUPPORTED
    assert _cum(lib, g, rp=None) == _lib.BSTA_ERR_NULL
    assert _cum(lib, g, ci=None) == _lib.BSTA_ERR_NULL
    assert _cum(lib, g, q=None) == _lib.BSTA_ERR_NULL
    assert _cum(lib, g, k=None) == _lib.BSTA_ERR_NULL
    assert _cum(lib, g, ws=None) == _lib.BSTA_ERR_NULL
    assert _cum(lib, g, flags=_lib.SELECT_PREPOOLED, q=None, k=None, ws=None) == _lib.BSTA_ERR_NULL
    assert "workspace" in _err(lib)
    need = 1 * 2 * 8 * 8
    assert _cum(lib, g, cap=need - 1) == _lib.BSTA_ERR_CAPACITY
    wsb = lib.attn_workspace_bytes(ctypes.byref(g), _lib.SELECT_CUMULATIVE)
    assert _cum(lib, g, wsb=wsb - 1) == _lib.BSTA_ERR_CAPACITY
    big = _g(T=64, Y=64, X=40)  # 16 * 16 * 10 = 2560 tiles, above one wave's 2048
    assert _cum(lib, big) == _lib.BSTA_ERR_SHAPE
    assert "2048" in _err(lib)
    assert lib.attn_geometry(ctypes.byref(_g(D=96)), None, None, None) == _lib.BSTA_ERR_UNSUPPORTED
    assert _cum(lib, _g(D=96)) == _lib.BSTA_ERR_UNSUPPORTED
    # attn_select_blocks does not take this mode (it has no threshold argument).
    assert _select(lib, g, mode=_lib.SELECT_CUMULATIVE) == _lib.BSTA_ERR_UNSUPPORTED
    assert "attn_select_cumulative" in _err(lib)


@pytest.mark.parametrize("grid", [(8, 8, 16), (21, 30, 52), (20, 48, 80), (5, 6, 7), (1, 1, 1)])
def test_geometry_tile128_matches_oracle(lib, grid):
    """4x4x8 (128-token) tiles: tile count, padded length and occupancy."""
    T, Y, X = grid
    t448 = geometry.TILE_SHAPES[128]
    g = _g(T=T, Y=Y, X=X, tile=t448)
    nt, lpad = ctypes.c_int32(), ctypes.c_int64()
    assert lib.attn_geometry(ctypes.byref(g), ctypes.byref(nt), ctypes.byref(lpad), None) == 0
    assert nt.value == geometry.num_tiles(T, Y, X, t448)
    assert lpad.value == geometry.padded_len(T, Y, X, t448)
    occ = (ctypes.c_int32 * nt.value)()
    assert lib.attn_geometry(ctypes.byref(g), None, None, occ) == 0
    assert np.array_equal(np.array(occ), geometry.occupancy(T, Y, X, t448))


def test_tile128_calls(lib):
    """The backward and query pruning take 128-token tiles: their argument
    checks pass up to the first check that fails before any HIP call (the
    workspace size, the keep ratio); other tile shapes are refused."""
    g = _g(tile=(4, 4, 8))
    assert lib.attn_prune_queries(ctypes.byref(g), FAKE, 1.5, FAKE, None, FAKE, None) == \
        _lib.BSTA_ERR_SHAPE
    assert lib.attn_prune_queries(ctypes.byref(g), FAKE, 0.5, None, None, FAKE, None) == \
        _lib.BSTA_ERR_NULL
    need = lib.attn_bwd_workspace_bytes(ctypes.byref(g), 16)
    assert need > 0
    assert _bwd(lib, g, wsb=need - 1) == _lib.BSTA_ERR_CAPACITY
    for bad in ((4, 4, 16), (4, 8, 4), (8, 4, 4), (2, 4, 8)):
        assert lib.attn_geometry(ctypes.byref(_g(tile=bad)), None, None, None) == _lib.BSTA_ERR_UNSUPPORTED


def test_pool_errors(lib):
    g = _g()
    assert lib.attn_pool(ctypes.byref(g), None, FAKE, None) == _lib.BSTA_ERR_NULL
    assert lib.attn_pool(ctypes.byref(g), FAKE, None, None) == _lib.BSTA_ERR_NULL
    assert lib.attn_pool(ctypes.byref(_g(D=32)), FAKE, FAKE, None) == _lib.BSTA_ERR_UNSUPPORTED


def test_prune_errors(lib):
    """Query pruning and the pruned forward check their arguments on the host."""
    g = _g()
    prune = lambda q=FAKE, ratio=0.5, km=FAKE, pq=FAKE, gg=g: lib.attn_prune_queries(  # noqa: E731
        ctypes.byref(gg), q, ratio, km, None, pq, None)
    for bad in (0.0, -0.5, 1.0000001, float("nan"), float("inf")):
        assert prune(ratio=bad) == _lib.BSTA_ERR_SHAPE, bad
        assert "keep_ratio" in _err(lib)
    assert prune(q=None) == _lib.BSTA_ERR_NULL
    assert prune(km=None) == _lib.BSTA_ERR_NULL
    assert prune(pq=None) == _lib.BSTA_ERR_NULL
    assert prune(gg=_g(D=96)) == _lib.BSTA_ERR_UNSUPPORTED
    scale = 1.0 / math.sqrt(g.D)
    fwd = lambda keep=FAKE, causal=0, sc=scale, q=FAKE: lib.attn_block_sparse_fwd_pruned(  # noqa: E731
        ctypes.byref(g), q, FAKE, FAKE, FAKE, FAKE, 16, sc, causal, keep, 1, FAKE, None, None)
    assert fwd(keep=None) == _lib.BSTA_ERR_NULL
    assert "keep_mask" in _err(lib)
    assert fwd(causal=1) == _lib.BSTA_ERR_UNSUPPORTED
    assert fwd(sc=0.5) == _lib.BSTA_ERR_UNSUPPORTED
    assert fwd(q=None) == _lib.BSTA_ERR_NULL


def _bwd(lib, g, scale=None, causal=0, ptrs=None, col_len=16, ws=FAKE, wsb=10 ** 12):
    if scale is None:
        scale = 1.0 / math.sqrt(g.D)
    p = [FAKE] * 11 if ptrs is None else ptrs
    return lib.attn_block_sparse_bwd(ctypes.byref(g), p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7],
                                     col_len, scale, causal, p[8], p[9], p[10], ws, wsb, None)


def test_bwd_workspace_and_errors(lib):
    g = _g(B=2, H=3, D=128, T=16, Y=48, X=80)
    nt = geometry.num_tiles(16, 48, 80)
    lpad = 64 * nt
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    # rowsum(dO*O) and log2(e)*lse per query slot, then the CSR transpose.
    want = up(up(up(2 * 2 * 3 * lpad * 4) + 2 * 3 * nt * 4) + 2 * 3 * nt * 4) + up(1000 * 4)
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(g), 1000) == want
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(g), -1) == _lib.BSTA_ERR_SHAPE
    s = _g()
    for n in range(11):
        ptrs = [FAKE] * 11
        ptrs[n] = None
        assert _bwd(lib, s, ptrs=ptrs) == _lib.BSTA_ERR_NULL, n
    assert _bwd(lib, s, ws=None) == _lib.BSTA_ERR_NULL
    assert _bwd(lib, s, causal=1) == _lib.BSTA_ERR_UNSUPPORTED
    assert _bwd(lib, s, scale=0.5) == _lib.BSTA_ERR_UNSUPPORTED
    assert _bwd(lib, s, col_len=-1) == _lib.BSTA_ERR_SHAPE
    need = lib.attn_bwd_workspace_bytes(ctypes.byref(s), 16)
    assert _bwd(lib, s, wsb=need - 1) == _lib.BSTA_ERR_CAPACITY
    big = _g(T=64, Y=64, X=68)  # 16 * 16 * 17 = 4352 tiles, above 4096
    assert _bwd(lib, big) == _lib.BSTA_ERR_SHAPE
    assert "4096" in _err(lib)


def _bwd_noalloc(lib, g, scale=None, causal=0, ptrs=None, col_len=16):
    if scale is None:
        scale = 1.0 / math.sqrt(g.D)
    p = [FAKE] * 11 if ptrs is None else ptrs
    return lib.attn_block_sparse_bwd_noalloc(ctypes.byref(g), p[0], p[1], p[2], p[3], p[4], p[5],
                                             p[6], p[7], col_len, scale, causal, p[8], p[9], p[10],
                                             None)


def test_bwd_noalloc_errors(lib):
    """The no-allocation backward checks its arguments as the workspace call
    does, and refuses a problem whose workspace exceeds its 64 MiB scratch
    on the host (every case here fails before any HIP call)."""
    s = _g()
    for n in range(11):
        ptrs = [FAKE] * 11
        ptrs[n] = None
        assert _bwd_noalloc(lib, s, ptrs=ptrs) == _lib.BSTA_ERR_NULL, n
    assert _bwd_noalloc(lib, s, causal=1) == _lib.BSTA_ERR_UNSUPPORTED
    assert _bwd_noalloc(lib, s, scale=0.5) == _lib.BSTA_ERR_UNSUPPORTED
    assert _bwd_noalloc(lib, s, col_len=-1) == _lib.BSTA_ERR_SHAPE
    big = _g(T=64, Y=64, X=68)
    assert _bwd_noalloc(lib, big) == _lib.BSTA_ERR_SHAPE
    # 64 MiB: the largest col_len whose workspace fits, and one entry more.
    limit = 64 << 20
    fixed = lib.attn_bwd_workspace_bytes(ctypes.byref(s), 0)
    fits = (limit - fixed) // 4
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(s), fits) <= limit
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(s), fits + 64) > limit
    assert _bwd_noalloc(lib, s, col_len=fits + 64) == _lib.BSTA_ERR_CAPACITY
    assert "64" in _err(lib) or "67108864" in _err(lib)


def _fwd(lib, g, scale=None, causal=0, q=FAKE, o=FAKE, rp=FAKE, col_len=16, fn="attn_block_sparse_fwd"):
    if scale is None:
        scale = 1.0 / math.sqrt(g.D)
    return getattr(lib, fn)(ctypes.byref(g), q, FAKE, FAKE, rp, FAKE, col_len, scale,
                            causal, o, None, None)


@pytest.mark.parametrize("fn", ["attn_block_sparse_fwd", "attn_block_sparse_fwd_raster"])
def test_fwd_errors(lib, fn):
    g = _g(D=128)
    assert _fwd(lib, g, causal=1, fn=fn) == _lib.BSTA_ERR_UNSUPPORTED
    assert "bidirectional" in _err(lib)
    assert _fwd(lib, g, scale=0.125, fn=fn) == _lib.BSTA_ERR_UNSUPPORTED
    assert _fwd(lib, g, scale=1.0, fn=fn) == _lib.BSTA_ERR_UNSUPPORTED
    assert _fwd(lib, g, scale=float("nan"), fn=fn) == _lib.BSTA_ERR_UNSUPPORTED
    assert _fwd(lib, g, q=None, fn=fn) == _lib.BSTA_ERR_NULL
    assert fn in _err(lib)
    assert _fwd(lib, g, o=None, fn=fn) == _lib.BSTA_ERR_NULL
    assert _fwd(lib, g, rp=None, fn=fn) == _lib.BSTA_ERR_NULL
    assert _fwd(lib, g, col_len=-1, fn=fn) == _lib.BSTA_ERR_SHAPE
    assert _fwd(lib, _g(D=80), fn=fn) == _lib.BSTA_ERR_UNSUPPORTED


def test_scale_tolerance_rule(lib):
    """Accept exactly the scales the pages' isclose(rel 1e-4, abs 1e-5) accepts
    (observed through the col_len error, which comes after the scale check)."""
    g = _g(D=128)
    exp = 1.0 / math.sqrt(128)
    for s, ok in [(exp * (1 + 5e-5), True), (exp * (1 + 3e-4), False), (exp - 9e-6, True),
                  (exp + 2e-5, False)]:
        st = _fwd(lib, g, scale=s, col_len=-1)
        assert st == (_lib.BSTA_ERR_SHAPE if ok else _lib.BSTA_ERR_UNSUPPORTED), s


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.attn_status_string(code)
    assert lib.attn_status_string(42) == b"unknown status"


def test_set_deterministic_returns_previous(lib):
    """Host-only switch: each call returns the previous mode (0 default walk,
    1 CSR order, 2 rotated everywhere; other values mean 1)."""
    first = lib.attn_set_deterministic(1)
    try:
        assert first in (0, 1, 2)
        assert lib.attn_set_deterministic(1) == 1
        assert lib.attn_set_deterministic(0) == 1
        assert lib.attn_set_deterministic(7) == 0
        assert lib.attn_set_deterministic(2) == 1
        assert lib.attn_set_deterministic(0) == 2
        assert lib.attn_set_deterministic(0) == 0
    finally:
        lib.attn_set_deterministic(first)


def test_key_walk_binding(lib):
    import block_sparse_tiled_amd as m
    first = m.attn_set_key_walk(m.WALK_ROTATED)
    try:
        assert m.attn_set_key_walk(m.WALK_CSR) == m.WALK_ROTATED
        assert m.attn_set_deterministic(False) is True
        assert m.attn_set_key_walk(m.WALK_AUTO) == m.WALK_AUTO
        with pytest.raises(ValueError):
            m.attn_set_key_walk(3)
    finally:
        m.attn_set_key_walk(first)


def test_binding_argument_errors_before_any_gpu_call():
    """The Python binding rejects bad combinations before it touches a GPU."""
    import block_sparse_tiled_amd as bsta
    g = bsta.Geometry(1, 2, 64, 8, 8, 8)
    with pytest.raises(ValueError, match="prepooled"):
        bsta.attn_select_cumulative(g, None, None, 0.5, prepooled=True)
    with pytest.raises(ValueError, match="threshold"):
        bsta._select_for(g, None, None, bsta.SELECT_CUMULATIVE, 0, None, None, 0)


# ------------------------------------------------------------------ packed sequences
PACKED_CASES = [
    ([5, (1, 2, 5), 3, (2, 2, 2)], (1, 1, 1)),
    ([7, (1, 4, 6), 70, (4, 4, 5)], (1, 1, 1)),
    ([0, (4, 8, 8), 7], (1, 2, 2)),
    ([(4, 4, 4), (4, 4, 8)], (1, 1, 1)),
    ([128, (20, 48, 80)], (1, 1, 1)),
    ([(5, 6, 7)], (1, 1, 1)),
]


def _pg(segs, patch=(1, 1, 1), B=1, H=2, D=64):
    return _lib.geom(B, H, D, 0, 0, 0, 4, segs, patch)


@pytest.mark.parametrize("segs,patch", PACKED_CASES)
def test_packed_geometry_matches_oracle(lib, segs, patch):
    """Tile count, padded length, per-tile occupancy, prefix, spans and
    packed length of a packed sequence against oracle/packed.py."""
    from oracle import packed
    lay = packed.layout(packed.token_segments(segs, patch))
    g = _pg(segs, patch)
    nt, lpad = ctypes.c_int32(), ctypes.c_int64()
    assert lib.attn_geometry(ctypes.byref(g), ctypes.byref(nt), ctypes.byref(lpad), None) == 0
    assert nt.value == len(lay["occ"])
    assert lpad.value == 64 * len(lay["occ"])
    occ = (ctypes.c_int32 * nt.value)()
    assert lib.attn_geometry(ctypes.byref(g), None, None, occ) == 0
    assert np.array_equal(np.array(occ), lay["occ"])
    npre, nreg, plen = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    spans = (ctypes.c_int32 * 32)()
    assert lib.attn_packed_info(ctypes.byref(g), ctypes.byref(npre), ctypes.byref(nreg), spans,
                                ctypes.byref(plen)) == 0
    assert npre.value == lay["num_prefix"]
    assert plen.value == lay["L"]
    assert [(spans[2 * r], spans[2 * r + 1]) for r in range(nreg.value)] == lay["spans"]


@pytest.mark.parametrize("segs,patch", PACKED_CASES[:4])
@pytest.mark.parametrize("sparsity,ref,exempt", [(0.5, 0.25, 1), (0.9, 0.1, 1), (0.0, None, 1),
                                                 (0.75, None, 0), (0.8, 1.0, 1), (1.0, 0.0, 1)])
def test_packed_capacity_matches_oracle(lib, segs, patch, sparsity, ref, exempt):
    """CSR entries of the packed selection: B*H times the oracle mask's
    entries of one head (row lengths do not depend on the scores)."""
    from oracle import packed
    lay = packed.layout(packed.token_segments(segs, patch))
    nt, R = len(lay["occ"]), len(lay["spans"])
    g = _pg(segs, patch, B=2, H=3)
    rk = float("nan") if ref is None else ref
    got = lib.attn_packed_capacity(ctypes.byref(g), sparsity, rk, exempt)
    if (not exempt and R != 1) or (exempt and R > 1 and ref is None):
        assert got in (_lib.BSTA_ERR_UNSUPPORTED, _lib.BSTA_ERR_SHAPE)
        return
    s = np.random.default_rng(7).standard_normal((1, 1, nt, nt))
    m = packed.select_mask(s, lay, sparsity, ref, exempt=bool(exempt))
    assert got == 2 * 3 * int(m.sum())


def test_packed_keep_count_double_precision(lib):
    """k = floor((1 - sparsity) * n) is taken in double precision as the
    oracle does: 1 - 0.9 is just below 0.1, so a 20-tile span keeps 1, not 2
    (a float32 sparsity would give 2)."""
    from oracle import packed
    segs = [(4, 20, 16)]                    # one region of 5 x 4 = 20 tiles
    g = _pg(segs, B=1, H=1)
    cap = lib.attn_packed_capacity(ctypes.byref(g), 0.9, float("nan"), 1)
    assert packed.keep_count(20, 1.0 - 0.9) == 1
    assert cap == 20 * 1


def test_packed_errors(lib):
    ok_segs = [5, (4, 4, 4)]
    bad_geoms = [
        ([(4, 7, 8)], (1, 2, 2)),           # latent side not a multiple of the patch
        ([12, 0], (1, 1, 1)),               # no video region
        ([(4, 4, 0)], (1, 1, 1)),           # empty region
        ([-1, (4, 4, 4)], (1, 1, 1)),       # negative rows
        ([(4, 4, 4)], (0, 1, 1)),           # patch 0
    ]
    for segs, patch in bad_geoms:
        assert lib.attn_geometry(ctypes.byref(_pg(segs, patch)), None, None, None) == _lib.BSTA_ERR_SHAPE
    g = _pg(ok_segs)
    g.segments.contents.kind[0] = 2          # unknown kind
    assert lib.attn_geometry(ctypes.byref(g), None, None, None) == _lib.BSTA_ERR_SHAPE
    g = _pg(ok_segs)
    g.segments.contents.count = 17
    assert lib.attn_geometry(ctypes.byref(g), None, None, None) == _lib.BSTA_ERR_SHAPE
    with pytest.raises(ValueError):
        _lib.segments([1] * 17)
    g = _pg(ok_segs)
    g.tile_x = 8                              # packed sequences use 64-token tiles
    assert lib.attn_geometry(ctypes.byref(g), None, None, None) == _lib.BSTA_ERR_UNSUPPORTED
    # single-grid geometry: no packed info, no packed selection
    assert lib.attn_packed_info(ctypes.byref(_g()), None, None, None, None) == _lib.BSTA_ERR_UNSUPPORTED
    assert lib.attn_packed_capacity(ctypes.byref(_g()), 0.5, 0.5, 1) == _lib.BSTA_ERR_UNSUPPORTED
    g = _pg([3, (4, 4, 4), (4, 4, 8)])
    nan = float("nan")
    for sp, rk, ex, want in [(nan, 0.5, 1, _lib.BSTA_ERR_SHAPE), (1.5, 0.5, 1, _lib.BSTA_ERR_SHAPE),
                             (0.5, nan, 1, _lib.BSTA_ERR_SHAPE), (0.5, 1.5, 1, _lib.BSTA_ERR_SHAPE),
                             (0.5, 0.5, 0, _lib.BSTA_ERR_UNSUPPORTED)]:
        assert lib.attn_packed_capacity(ctypes.byref(g), sp, rk, ex) == want
    cap = lib.attn_packed_capacity(ctypes.byref(g), 0.5, 0.5, 1)
    ws = lib.attn_workspace_bytes(ctypes.byref(g), _lib.SELECT_TOPK)
    assert cap > 0 and ws > 0

    def sel(flags=0, q=FAKE, k=FAKE, rp=FAKE, ci=FAKE, cap_=cap, w=FAKE, wsb=ws, geom=g):
        return lib.attn_select_packed(ctypes.byref(geom), q, k, flags, 0.5, 0.5, 1, None, rp, ci,
                                      cap_, w, wsb, None)
    assert sel(rp=None) == _lib.BSTA_ERR_NULL
    assert sel(q=None) == _lib.BSTA_ERR_NULL
    assert sel(w=None) == _lib.BSTA_ERR_NULL
    assert sel(flags=7) == _lib.BSTA_ERR_UNSUPPORTED
    assert sel(cap_=cap - 1) == _lib.BSTA_ERR_CAPACITY
    assert sel(wsb=ws - 1) == _lib.BSTA_ERR_CAPACITY
    assert sel(geom=_g()) == _lib.BSTA_ERR_UNSUPPORTED
    # window mode and query pruning take a single grid
    w = (ctypes.c_int32 * 6)(1, 1, 1, 1, 1, 1)
    assert lib.attn_select_capacity(ctypes.byref(_pg(ok_segs)), _lib.SELECT_STA, 0, w) == \
        _lib.BSTA_ERR_UNSUPPORTED
    assert lib.attn_prune_queries(ctypes.byref(_pg(ok_segs)), FAKE, 0.5, FAKE, None, FAKE, None) == \
        _lib.BSTA_ERR_UNSUPPORTED
    scale = 1.0 / math.sqrt(64)
    assert lib.attn_block_sparse_fwd_pruned(ctypes.byref(_pg(ok_segs)), FAKE, FAKE, FAKE, FAKE, FAKE, 16,
                                            scale, 0, FAKE, 1, FAKE, None, None) == _lib.BSTA_ERR_UNSUPPORTED


def test_packed_python_geometry(lib):
    """Geometry.packed: L and the layout come from the library."""
    import block_sparse_tiled_amd as m
    from oracle import packed
    segs = [5, (1, 2, 5), 3, (2, 2, 2)]
    g = m.Geometry.packed(1, 2, 64, segs)
    lay = packed.layout(packed.token_segments(segs))
    assert g.L == lay["L"] and g.num_tiles == len(lay["occ"]) and g.Lpad == 64 * len(lay["occ"])
    info = m.attn_packed_info(g)
    assert info["num_prefix"] == lay["num_prefix"] and info["spans"] == lay["spans"]
    assert m.attn_packed_capacity(g, 0.5, 0.5) == 2 * int(
        packed.select_mask(np.zeros((1, 1, 5, 5)), lay, 0.5, 0.5).sum())
