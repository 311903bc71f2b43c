"""GPU parity of query pruning (attn_prune_queries, attn_block_sparse_fwd_pruned)
against the CPU oracle (oracle/prune.py, reading R21).

Bars: kept counts exact; kept sets equal to the oracle's except in tiles
whose keep-boundary score gap is below PRUNE_BAND, where they may differ
only among tokens within that band of the boundary; kept means within
1e-5*(1+|x|) of the oracle's means of the GPU's (validated) kept rows; the
selection by the top-k / cumulative rules of the oracle on those means;
kept rows' outputs within max-abs 2e-2 / mean-abs 2e-3 of the oracle's
attention under the GPU's selection; pruned and pad rows exactly +0.0.
"""
import math

import numpy as np
import pytest

import workloads
from oracle import geometry, prune, select, tiling
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

PRUNE_BAND = 1e-5

CASES = {
    "ragged_d128": (workloads.custom("prune_ragged_d128", 2, 3, 128, 5, 6, 7, "topk", 3, seed=71), 0.5),
    "ragged_d64": (workloads.custom("prune_ragged_d64", 1, 2, 64, 9, 13, 10, "topk", 5, seed=72), 0.3),
    "smooth_40": (workloads.custom("prune_smooth_40", 1, 4, 128, 8, 16, 20, "topk", 10, "smooth",
                                   seed=73), 0.5),
    "one_token": (workloads.custom("prune_one_token", 1, 1, 128, 1, 1, 1, "topk", 1, seed=74), 0.2),
}


@pytest.fixture(scope="module")
def bsta():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    import block_sparse_tiled_amd as m
    from block_sparse_tiled_amd import _lib
    _lib.load()
    return m


T448 = geometry.TILE_SHAPES[128]


def _bits(keep_dev, E=64):
    """int64 [B, H, Nt * E/64] device mask words (one per 64-slot unit) ->
    bool [B, H, Nt, E]."""
    words = keep_dev.cpu().numpy().view(np.uint64)
    bits = ((words[..., None] >> np.arange(64, dtype=np.uint64)) & np.uint64(1)).astype(bool)
    B, Hh, nu, _ = bits.shape
    return bits.reshape(B, Hh, nu * 64 // E, E)


def accept_keep(gpu_keep, qt, T, Y, X, ratio, tile=geometry.TILE):
    """Every tile's kept set against the oracle (module docstring).  Returns
    (tiles equal to the oracle's, tiles inside the band)."""
    want = prune.keep_mask(qt, T, Y, X, ratio, tile)
    occ = geometry.occupancy(T, Y, X, tile)
    E = geometry.tile_elems(tile)
    B, _, Hh, _ = qt.shape
    same = band = 0
    for b in range(B):
        for h in range(Hh):
            for j, n in enumerate(occ):
                g, o = gpu_keep[b, h, j], want[b, h, j]
                assert not g[n:].any(), f"tile {(b, h, j)}: a pad slot is kept"
                assert g.sum() == prune.kept_count(int(n), ratio), f"tile {(b, h, j)}: count"
                if np.array_equal(g, o):
                    same += 1
                    continue
                s = prune.redundancy(qt[b, j * E:j * E + n, h])
                hi_kept, lo_pruned = s[o[:n]].max(), s[~o[:n]].min()
                assert lo_pruned - hi_kept < PRUNE_BAND, f"tile {(b, h, j)}: sets differ, gap {lo_pruned - hi_kept}"
                diff = np.nonzero(g[:n] != o[:n])[0]
                assert np.all(s[diff] >= hi_kept - PRUNE_BAND) and np.all(s[diff] <= lo_pruned + PRUNE_BAND)
                band += 1
    return same, band


def _run(m, w, inp, ratio, mode, threshold=0.5, min_blocks=1, raster=True, tile_x=4):
    """Tile Q (plain) and K (pooled into the selection), prune Q into the
    selection's pooled-Q part, select from the kept means, attend."""
    import torch
    g = m.Geometry(w.B, w.H, w.D, w.T, w.Y, w.X, tile_x=tile_x)
    q, k, v = (H.to_dev(inp[n]) for n in ("q", "k", "v"))
    smode = m.SELECT_CUMULATIVE if mode == "cumulative" else m.SELECT_TOPK
    sel = m.attn_select_alloc(g, smode, w.topk, want_mask=True)
    pq, pk = sel.pooled(g)
    qt = m.attn_tile(g, q)
    kt = m.attn_tile_pool(g, k, pk)
    vt = m.attn_tile(g, v)
    keep, count, _ = m.attn_prune_queries(g, qt, ratio, pooled=pq)
    if mode == "cumulative":
        m.attn_select_cumulative(g, None, None, threshold, min_blocks, prepooled=True, out=sel)
    else:
        m.attn_select_blocks(g, None, None, m.SELECT_TOPK | m.SELECT_PREPOOLED, w.topk, out=sel)
    rows = w.L if raster else g.Lpad
    o = torch.full((w.B, rows, w.H, w.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    o, lse = m.attn_block_sparse_fwd(g, qt, kt, vt, sel.row_ptr, sel.col_idx, out=o, want_lse=True,
                                     raster=raster, keep=keep)
    torch.cuda.synchronize()
    return dict(g=g, qt=qt, kt=kt, vt=vt, sel=sel, keep=keep, count=count, o=o, lse=lse)


def _check(w, inp, r, ratio, mode, threshold=0.5, min_blocks=1, heads=None, tiles=None,
           tile=geometry.TILE):
    """The GPU's pruning, selection and output against the oracle."""
    T, Y, X = w.T, w.Y, w.X
    E = geometry.tile_elems(tile)
    tf = {n: workloads.bf16_to_f32(tiling.tile(inp[n], T, Y, X, tile)) for n in ("q", "k", "v")}
    gkeep = _bits(r["keep"], E)
    same, band = accept_keep(gkeep, tf["q"], T, Y, X, ratio, tile)
    H.log(f"  kept sets: {same} equal, {band} inside the band")
    occ = geometry.occupancy(T, Y, X, tile)
    want_count = np.array([prune.kept_count(int(n), ratio) for n in occ])
    assert np.array_equal(r["count"].cpu().numpy(), np.broadcast_to(want_count, r["count"].shape))
    # means of the GPU's kept rows, and the keys' means
    opq = prune.pool_kept(tf["q"], gkeep)
    opk = select.pool(tf["k"], T, Y, X, tile)
    gpq, gpk = (t.cpu().numpy() for t in r["sel"].pooled(r["g"]))
    assert np.all(np.abs(gpq - opq) <= H.POOL_TOL * (1 + np.abs(opq)))
    assert np.all(np.abs(gpk - opk) <= H.POOL_TOL * (1 + np.abs(opk)))
    s = select.scores(opq, opk)
    gmask = r["sel"].block_mask.cpu().numpy().astype(bool)
    if mode == "cumulative":
        H.accept_cumulative_rows(gmask, s, w.D, threshold, min_blocks)
    else:
        H.accept_topk_rows(gmask, s, w.topk)
    nt = len(occ)
    hs = range(w.H) if heads is None else heads
    js = range(nt) if tiles is None else tiles
    rows = [(b, h, i) for b in range(w.B) for h in hs for i in js]
    ref, rlse = prune.pruned_attention(tf["q"], tf["k"], tf["v"], gmask, gkeep, T, Y, X,
                                       1.0 / math.sqrt(w.D), rows, tile)
    got = H.bf16_dev_to_f32(r["o"])
    assert not np.isnan(got).any(), "every raster row is written"
    order = geometry.tile_order(T, Y, X, tile)
    start = np.concatenate([[0], np.cumsum(occ)])
    kept_g, kept_r = [], []
    for b, h, i in rows:
        toks = order[start[i]:start[i + 1]]
        k = gkeep[b, h, i, :occ[i]]
        assert np.all(got[b, toks[~k], h] == 0.0), "pruned rows are +0.0"
        kept_g.append(got[b, toks[k], h])
        kept_r.append(ref[b, i * E + np.nonzero(k)[0], h])
    mx, mean = H.compare_outputs(np.concatenate(kept_g), np.concatenate(kept_r), "kept rows")
    H.log(f"  kept rows max-abs {mx:.3g}, mean-abs {mean:.3g}")
    glse = r["lse"].cpu().numpy()
    for b, h, i in rows:
        k = gkeep[b, h, i]
        sl = i * E + np.arange(E)
        assert np.all(np.isneginf(glse[b, h, sl[~k]]))
        assert np.abs(glse[b, h, sl[k]] - rlse[b, h, sl[k]]).max() <= H.LSE_TOL


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("mode", ["cumulative", "topk"])
def test_pruned_path(bsta, name, mode):
    w, ratio = CASES[name]
    H.log(f"pruned path {name} ({mode}, ratio {ratio})")
    inp = H.inputs(w)
    r = _run(bsta, w, inp, ratio, mode)
    _check(w, inp, r, ratio, mode)


def test_pruned_tiled_output(bsta):
    """The tiled-output variant writes the same rows as the raster one, in
    slot order, with pad and pruned slots zero."""
    w, ratio = CASES["ragged_d128"]
    inp = H.inputs(w)
    prev = bsta.attn_set_deterministic(True)
    try:
        a = _run(bsta, w, inp, ratio, "cumulative", raster=True)
        b = _run(bsta, w, inp, ratio, "cumulative", raster=False)
    finally:
        bsta.attn_set_deterministic(prev)
    untiled = tiling.untile(H.from_dev(b["o"]), w.T, w.Y, w.X)
    assert np.array_equal(H.from_dev(a["o"]), untiled)


def test_ratio_one_is_the_unpruned_path(bsta):
    """Keeping every token: all valid bits set, the kept means equal
    attn_tile_pool's pooled Q bit for bit, and the pruned forward equals the
    plain one bit for bit (CSR-order walk)."""
    import torch
    w, _ = CASES["smooth_40"]
    inp = H.inputs(w)
    g = bsta.Geometry(w.B, w.H, w.D, w.T, w.Y, w.X)
    prev = bsta.attn_set_deterministic(True)
    try:
        r = _run(bsta, w, inp, 1.0, "topk")
        sel = bsta.attn_select_alloc(g, bsta.SELECT_TOPK, w.topk, want_mask=False)
        pq, _ = sel.pooled(g)
        bsta.attn_tile_pool(g, H.to_dev(inp["q"]), pq)
        o = bsta.attn_block_sparse_fwd(g, r["qt"], r["kt"], r["vt"], r["sel"].row_ptr,
                                       r["sel"].col_idx, raster=True)
        torch.cuda.synchronize()
    finally:
        bsta.attn_set_deterministic(prev)
    occ = geometry.occupancy(w.T, w.Y, w.X)
    full = np.arange(64)[None, :] < occ[:, None]
    assert np.array_equal(_bits(r["keep"]), np.broadcast_to(full, _bits(r["keep"]).shape))
    assert torch.equal(r["sel"].pooled(g)[0].view(torch.int32), pq.view(torch.int32))
    assert torch.equal(r["o"].view(torch.int16), o.view(torch.int16))


@pytest.mark.timeout(900)
def test_pruned_full_size_c3(bsta):
    """The 40-head 76,800-token workload with half the queries pruned and the
    cumulative threshold: every tile's kept set and count, every pooled
    vector, the selection rows of two heads, and the kept rows of one query
    tile per head plus every tile of one head."""
    w = workloads.WORKLOADS["c3"]
    ratio, tau = 0.5, 0.15
    H.log("pruned c3: generating inputs")
    inp = H.inputs(w)
    r = _run(bsta, w, inp, ratio, "cumulative", threshold=tau, min_blocks=0)
    T, Y, X = w.T, w.Y, w.X
    tf = {n: workloads.bf16_to_f32(tiling.tile(inp[n], T, Y, X)) for n in ("q", "k", "v")}
    H.log("pruned c3: kept sets")
    gkeep = _bits(r["keep"])
    same, band = accept_keep(gkeep, tf["q"], T, Y, X, ratio)
    H.log(f"  kept sets: {same} equal, {band} inside the band")
    assert np.all(r["count"].cpu().numpy() == 32)
    opq = prune.pool_kept(tf["q"], gkeep)
    gpq = r["sel"].pooled(r["g"])[0].cpu().numpy()
    assert np.all(np.abs(gpq - opq) <= H.POOL_TOL * (1 + np.abs(opq)))
    opk = select.pool(tf["k"], T, Y, X)
    gmask = r["sel"].block_mask.cpu().numpy().astype(bool)
    heads = [3, 29]
    s = select.scores(opq[:, heads], opk[:, heads])
    H.accept_cumulative_rows(gmask[:, heads], s, w.D, tau, 0)
    nt = geometry.num_tiles(T, Y, X)
    rng = np.random.default_rng(77)
    rows = [(0, h, int(rng.integers(nt))) for h in range(w.H)] + [(0, 11, i) for i in range(nt)]
    H.log(f"pruned c3: oracle attention on {len(rows)} query tiles")
    ref, _ = prune.pruned_attention(tf["q"], tf["k"], tf["v"], gmask, gkeep, T, Y, X,
                                    1.0 / math.sqrt(w.D), rows)
    got = H.bf16_dev_to_f32(r["o"])
    assert not np.isnan(got).any()
    occ = geometry.occupancy(T, Y, X)
    order = geometry.tile_order(T, Y, X)
    kept_g, kept_r = [], []
    for b, h, i in rows:
        toks = order[i * 64:(i + 1) * 64]
        k = gkeep[b, h, i, :occ[i]]
        assert np.all(got[b, toks[~k], h] == 0.0)
        kept_g.append(got[b, toks[k], h])
        kept_r.append(ref[b, i * 64 + np.nonzero(k)[0], h])
    mx, mean = H.compare_outputs(np.concatenate(kept_g), np.concatenate(kept_r), "kept rows")
    H.log(f"  kept rows max-abs {mx:.3g}, mean-abs {mean:.3g}")


CASES128 = {
    "ragged_d128": (workloads.custom("prune128_ragged_d128", 2, 3, 128, 5, 6, 19, "topk", 2, seed=81),
                    0.5),
    "ragged_d64": (workloads.custom("prune128_ragged_d64", 1, 2, 64, 9, 13, 10, "topk", 3, seed=82),
                   0.3),
}


@pytest.mark.parametrize("name", sorted(CASES128))
@pytest.mark.parametrize("mode", ["cumulative", "topk"])
def test_pruned_path_tile128(bsta, name, mode):
    """128-token tiles: each tile keeps kept_count(n) of its up to 128 tokens
    (two mask words, one per 64-slot unit), selection from the kept means,
    kept rows against the oracle run with the same tile shape."""
    w, ratio = CASES128[name]
    H.log(f"pruned path, 128-token tiles, {name} ({mode}, ratio {ratio})")
    inp = H.inputs(w)
    r = _run(bsta, w, inp, ratio, mode, tile_x=8)
    _check(w, inp, r, ratio, mode, tile=T448)


def test_ratio_one_is_the_unpruned_path_tile128(bsta):
    """128-token tiles at ratio 1: every valid bit set, and the kept means
    equal attn_tile_pool's pooled Q bit for bit (the same sixteen runs of
    eight slots, added in order)."""
    import torch
    w, _ = CASES128["ragged_d128"]
    inp = H.inputs(w)
    r = _run(bsta, w, inp, 1.0, "topk", tile_x=8)
    g = r["g"]
    sel = bsta.attn_select_alloc(g, bsta.SELECT_TOPK, w.topk, want_mask=False)
    pq, _ = sel.pooled(g)
    bsta.attn_tile_pool(g, H.to_dev(inp["q"]), pq)
    torch.cuda.synchronize()
    occ = geometry.occupancy(w.T, w.Y, w.X, T448)
    full = np.arange(128)[None, :] < occ[:, None]
    got = _bits(r["keep"], 128)
    assert np.array_equal(got, np.broadcast_to(full, got.shape))
    assert torch.equal(r["sel"].pooled(g)[0].view(torch.int32), pq.view(torch.int32))
