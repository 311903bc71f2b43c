"""Pins of the packed multi-region oracle (oracle/packed.py, reading R24)
against things other than itself: a hand-derived layout, a hand-derived
selection, the single-region case against the single-grid path, the
all-dense case against torch's attention, a token-level brute force, and
the page's argument checks."""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import geometry, packed, pipeline, select, tiling

SEGS = [5, (1, 2, 5), 3, (2, 2, 2)]


def test_layout_golden():
    """Hand-derived: dense 5 rows (tokens 0-4), region 1x2x5 (5-14), dense 3
    rows (15-17), region 2x2x2 (18-25).  Prefix tiles: [0..4], [15..17].
    Region 1: tile (0,0,0) holds x 0..3 of both y rows -> 5,6,7,8,10,11,12,13;
    tile (0,0,1) holds x 4 -> 9, 14.  Region 2: one tile, 18..25."""
    lay = packed.layout(packed.token_segments(SEGS))
    assert lay["L"] == 26
    assert lay["num_prefix"] == 2
    assert lay["spans"] == [(2, 4), (4, 5)]
    assert list(lay["occ"]) == [5, 3, 8, 2, 8]
    st = lay["slot_token"]
    want = [list(range(0, 5)), [15, 16, 17], [5, 6, 7, 8, 10, 11, 12, 13], [9, 14], list(range(18, 26))]
    for j, toks in enumerate(want):
        assert list(st[j * 64:j * 64 + len(toks)]) == toks
        assert np.all(st[j * 64 + len(toks):(j + 1) * 64] == -1)


def test_token_segments_and_errors():
    assert packed.token_segments([0, (4, 8, 8), 7], patch=(1, 2, 2)) == [(4, 4, 4), 7]
    with pytest.raises(ValueError):
        packed.token_segments([(4, 7, 8)], patch=(1, 2, 2))     # 7 not a multiple of 2
    with pytest.raises(ValueError):
        packed.token_segments([12, 0])                          # no video region
    lay = packed.layout(packed.token_segments([(4, 4, 4), (4, 4, 8)]))
    with pytest.raises(ValueError):
        packed.span_keeps(lay, 0.5)                             # reference region, no keep rate
    with pytest.raises(ValueError):
        packed.select_mask(np.zeros((1, 1, 3, 3)), lay, 0.5, 0.5, exempt=False)


def test_keep_count_golden():
    # floor(keep*n) clamped to [1, n]: 0.1*10 = 1; 0.25*8 = 2; 0.05*8 = 0.4 -> 1; 1.0*5 = 5; 0.99*3 = 2
    for n, keep, k in [(10, 0.1, 1), (8, 0.25, 2), (8, 0.05, 1), (5, 1.0, 5), (3, 0.99, 2)]:
        assert packed.keep_count(n, keep) == k


def test_selection_golden():
    """Prefix of one tile, a reference span of 3 tiles (keep 1/3 -> 1) and a
    generated span of 4 tiles (sparsity 0.5 -> 2).  Scores of video query
    tile 1 against tiles 0..7: [9, 1, 5, 3, 2, 7, 7, 0] -> prefix {0}, span
    1..3 best {2} (5), span 4..7 best two {5, 6} (7, 7).  Prefix query tile 0
    keeps all."""
    lay = {"num_prefix": 1, "spans": [(1, 4), (4, 8)]}
    s = np.zeros((1, 1, 8, 8))
    s[0, 0, 1] = [9, 1, 5, 3, 2, 7, 7, 0]
    s[0, 0, 4] = [0, 4, 4, 4, 1, 1, 1, 1]      # ties: lower index wins
    m = packed.select_mask(s, lay, 0.5, ref_keep_rate=1 / 3)
    assert m[0, 0, 0].all()
    assert list(np.nonzero(m[0, 0, 1])[0]) == [0, 2, 5, 6]
    assert list(np.nonzero(m[0, 0, 4])[0]) == [0, 1, 4, 5]
    assert (m[0, 0, 1:].sum(-1) == 4).all()
    # compete: one region; k = floor(0.5 * 8) = 4 over all tiles
    lay1 = {"num_prefix": 1, "spans": [(1, 8)]}
    mc = packed.select_mask(s, lay1, 0.5, exempt=False)
    assert list(np.nonzero(mc[0, 0, 1])[0]) == [0, 2, 5, 6]
    assert (mc.sum(-1) == 4).all()
    # sparsity 0: every tile
    assert packed.select_mask(s, lay, 0.0, ref_keep_rate=0.3).all()


def test_single_region_is_the_single_grid_path():
    """No dense segment and one region: the packed layout is the grid's, and
    the exempt selection is the grid's top-k with k = floor((1 - s) * Nt)."""
    w = workloads.custom("packed_single", 1, 2, 64, 5, 6, 7, "topk", 3, seed=101)
    inp = workloads.make_inputs(w)
    lay = packed.layout(packed.token_segments([(w.T, w.Y, w.X)]))
    slots = geometry.token_slots(w.T, w.Y, w.X)
    assert np.array_equal(lay["slot_token"][slots], np.arange(w.L))
    assert np.array_equal(lay["occ"], geometry.occupancy(w.T, w.Y, w.X))
    nt = geometry.num_tiles(w.T, w.Y, w.X)
    sparsity = 0.75
    k = packed.keep_count(nt, 1 - sparsity)
    f = {n: pipeline.widen(inp[n]) for n in ("q", "k", "v")}
    r = packed.run(f["q"], f["k"], f["v"], [(w.T, w.Y, w.X)], sparsity=sparsity)
    ref = pipeline.run(inp["q"], inp["k"], inp["v"], w.T, w.Y, w.X, "topk", k)
    assert np.array_equal(r["mask"], ref["mask"])
    assert np.allclose(r["out"], ref["out"], rtol=0, atol=1e-12)


def test_dense_build_is_full_attention():
    """Sparsity 0 keeps every tile: plain softmax attention over the whole
    packed sequence (torch, float64)."""
    rng = np.random.default_rng(102)
    segs = [7, (1, 4, 6), 70, (4, 4, 5)]
    L = packed.layout(packed.token_segments(segs))["L"]
    q, k, v = (rng.standard_normal((1, L, 2, 16)) for _ in range(3))
    r = packed.run(q, k, v, segs, sparsity=0.0, ref_keep_rate=0.5)
    assert r["mask"].all()
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x.transpose(0, 2, 1, 3)) for x in (q, k, v))).numpy().transpose(0, 2, 1, 3)
    assert np.allclose(r["out"], ref, rtol=0, atol=1e-10)


def test_token_level_brute_force():
    """Every packed token's output equals softmax attention over the tokens of
    the tiles its tile selected, built token by token from the mask."""
    rng = np.random.default_rng(103)
    segs = [9, (2, 4, 6), (3, 5, 4)]
    lay = packed.layout(packed.token_segments(segs))
    L = lay["L"]
    q, k, v = (rng.standard_normal((1, L, 1, 8)) for _ in range(3))
    r = packed.run(q, k, v, segs, sparsity=0.6, ref_keep_rate=0.5)
    tile_of = np.empty(L, dtype=np.int64)
    valid = lay["slot_token"] >= 0
    tile_of[lay["slot_token"][valid]] = np.nonzero(valid)[0] // 64
    mask = r["mask"][0, 0]
    for l in range(L):
        keys = np.nonzero(mask[tile_of[l]][tile_of])[0]
        s = q[0, l, 0] @ k[0, keys, 0].T / math.sqrt(8)
        p = np.exp(s - s.max())
        want = p @ v[0, keys, 0] / p.sum()
        assert np.allclose(r["out"][0, l, 0], want, rtol=0, atol=1e-12)
    # tile / untile round trip and zero pads
    qt = packed.tile(q, lay)
    assert np.array_equal(packed.untile(qt, lay), q)
    assert np.all(qt[:, ~valid] == 0)


def test_pool_matches_grouped_sums():
    rng = np.random.default_rng(104)
    segs = [70, (2, 3, 9)]
    lay = packed.layout(packed.token_segments(segs))
    x = rng.standard_normal((1, lay["L"], 2, 4))
    tile_of = np.empty(lay["L"], dtype=np.int64)
    valid = lay["slot_token"] >= 0
    tile_of[lay["slot_token"][valid]] = np.nonzero(valid)[0] // 64
    sums = np.zeros((len(lay["occ"]), 2, 4))
    np.add.at(sums, tile_of, x[0])
    want = (sums / np.bincount(tile_of)[:, None, None]).astype(np.float32).transpose(1, 0, 2)
    assert np.array_equal(packed.pool(packed.tile(x, lay), lay)[0], want)


def test_backward_against_autograd():
    """The packed gradients equal torch autograd (float64) of softmax
    attention over the packed tokens under the token mask the tile mask
    implies, on a prefix plus two regions with ragged tiles."""
    rng = np.random.default_rng(105)
    segs = [9, (2, 4, 6), (3, 5, 4)]
    lay = packed.layout(packed.token_segments(segs))
    L = lay["L"]
    q, k, v, do = (rng.standard_normal((1, L, 2, 8)) for _ in range(4))
    r = packed.run(q, k, v, segs, sparsity=0.6, ref_keep_rate=0.5)
    dot = packed.tile(do, lay)
    dq, dk, dv = packed.attention_backward(r["qt"], r["kt"], r["vt"], dot, r["mask"], lay)
    tile_of = np.empty(L, dtype=np.int64)
    valid = lay["slot_token"] >= 0
    tile_of[lay["slot_token"][valid]] = np.nonzero(valid)[0] // 64
    tq, tk, tv = (torch.from_numpy(x.transpose(0, 2, 1, 3).copy()).requires_grad_() for x in (q, k, v))
    allowed = torch.from_numpy(r["mask"][0][:, tile_of][:, :, tile_of])          # [H, L, L]
    s = tq @ tk.transpose(-1, -2) / math.sqrt(8)
    s = s.masked_fill(~allowed[None], float("-inf"))
    out = torch.softmax(s, dim=-1) @ tv
    (out * torch.from_numpy(do.transpose(0, 2, 1, 3))).sum().backward()
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        want = ref.numpy().transpose(0, 2, 1, 3)
        assert np.allclose(packed.untile(got, lay), want, rtol=0, atol=1e-12)
        assert np.all(got[:, ~valid] == 0)


def test_backward_single_region_is_the_grid_backward():
    """One region, no dense segment: the grid backward of the single-grid
    oracle on the same mask."""
    from oracle import attention as oatt
    rng = np.random.default_rng(106)
    T, Y, X = 5, 6, 7
    lay = packed.layout(packed.token_segments([(T, Y, X)]))
    nt = len(lay["occ"])
    qt, kt, vt, dot = (packed.tile(rng.standard_normal((1, T * Y * X, 2, 16)), lay) for _ in range(4))
    mask = rng.random((1, 2, nt, nt)) < 0.5
    mask[..., 0] = True
    got = packed.attention_backward(qt, kt, vt, dot, mask, lay)
    ref = oatt.block_sparse_attention_backward(qt, kt, vt, dot, mask, T, Y, X)
    for a, b in zip(got, ref):
        assert np.allclose(a, b, rtol=0, atol=1e-12)
