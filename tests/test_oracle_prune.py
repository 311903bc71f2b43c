"""Pins of the query-pruning oracle (oracle/prune.py) against things other
than itself: hand-derived fixtures (tests/golden/prune_examples.json), the
cosine written through angles for 2-D data, invariances of the redundancy
score, the keep-everything case reducing to the unpruned path, and kept rows
against a dense brute force with an explicit token mask."""
import json
import math
import os

import numpy as np
import pytest

import workloads
from oracle import attention, geometry, pipeline, prune, select, tiling

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "prune_examples.json")) as f:
        return json.load(f)


def _tiled(rows, grid):
    """[L, D] raster rows -> tiled [1, Lpad, 1, D]."""
    T, Y, X = grid
    x = np.asarray(rows, dtype=np.float64)[None, :, None, :]
    return tiling.tile(x, T, Y, X)


def test_kept_count_golden():
    for n, ratio, c in _golden()["kept_counts"]["cases"]:
        assert prune.kept_count(n, ratio) == c, (n, ratio)
    for bad in (0.0, -0.1, 1.01, float("nan")):
        with pytest.raises(ValueError):
            prune.kept_count(8, bad)
    assert prune.kept_count(0, 0.5) == 0


def test_tile_2x2_golden():
    g = _golden()["tile_2x2"]
    qt = _tiled(g["q_rows"], g["grid"])
    assert np.allclose(prune.redundancy(qt[0, :4, 0]), g["scores"], rtol=0, atol=1e-15)
    for ratio, kept in g["kept"].items():
        keep = prune.keep_mask(qt, *g["grid"], float(ratio))
        assert list(np.nonzero(keep[0, 0, 0])[0]) == kept, ratio
        pq = prune.pool_kept(qt, keep)
        assert np.array_equal(pq[0, 0, 0], np.array(g["pooled_kept"][ratio], dtype=np.float32))


def test_ragged_golden():
    g = _golden()["ragged_1x1x5"]
    qt = _tiled(g["q_rows"], g["grid"])
    keep = prune.keep_mask(qt, *g["grid"], g["ratio"])
    assert list(np.nonzero(keep[0, 0, 0])[0]) == g["kept_tile0"]
    assert list(np.nonzero(keep[0, 0, 1])[0]) == g["kept_tile1"]
    assert not keep[0, 0, 1, 1:].any(), "pad slots are never kept"
    assert np.array_equal(prune.pool_kept(qt, keep)[0, 0], np.array(g["pooled_kept"], dtype=np.float32))


def test_redundancy_against_angles():
    """For 2-D rows cos(q, m) = cos(angle(q) - angle(m)), computed from atan2."""
    rng = np.random.default_rng(61)
    for _ in range(50):
        q = rng.standard_normal((int(rng.integers(2, 9)), 2))
        m = q.mean(axis=0)
        want = np.cos(np.arctan2(q[:, 1], q[:, 0]) - np.arctan2(m[1], m[0]))
        assert np.allclose(prune.redundancy(q), want, rtol=0, atol=1e-12)


def test_redundancy_invariances():
    rng = np.random.default_rng(62)
    assert np.all(np.abs(prune.redundancy(rng.standard_normal((40, 16)))) <= 1 + 1e-12)
    # rows along one direction (any positive lengths) all point the mean's way
    same = np.tile(rng.standard_normal(16), (8, 1)) * rng.uniform(0.5, 2.0, size=(8, 1))
    assert np.allclose(prune.redundancy(same), 1.0, atol=1e-12)
    assert np.allclose(prune.redundancy(np.zeros((5, 4))), 0.0)
    # a row pointing against the mean scores -1
    q2 = np.array([[1.0, 0.0], [1.0, 0.0], [1.0, 0.0], [-0.5, 0.0]])
    assert np.isclose(prune.redundancy(q2)[3], -1.0)
    # the score does not depend on a row's length (mean held fixed by a
    # compensating row): scale row 0 by 3 and row 1 so the sum is unchanged
    q3 = rng.standard_normal((6, 5))
    q4 = q3.copy()
    q4[0] *= 3.0
    q4[1] -= 2.0 * q3[0]
    assert np.isclose(prune.redundancy(q4)[0], prune.redundancy(q3)[0], rtol=0, atol=1e-12)


def test_keep_mask_order_and_ties():
    """Kept tokens score no higher than pruned ones, counts follow kept_count,
    and equal scores are decided toward the lower slot."""
    rng = np.random.default_rng(63)
    T, Y, X = 5, 6, 7
    qt = tiling.tile(rng.standard_normal((2, T * Y * X, 3, 8)), T, Y, X)
    occ = geometry.occupancy(T, Y, X)
    for ratio in (0.1, 0.5, 0.77, 1.0):
        keep = prune.keep_mask(qt, T, Y, X, ratio)
        for b in range(2):
            for h in range(3):
                for j, n in enumerate(occ):
                    k = keep[b, h, j]
                    assert k.sum() == prune.kept_count(int(n), ratio)
                    assert not k[n:].any()
                    s = prune.redundancy(qt[b, j * 64:j * 64 + n, h])
                    if k[:n].all():
                        continue
                    assert s[k[:n]].max() <= s[~k[:n]].min()
    # ties: four identical rows and one opposite row in a 1x1x5 grid (tile 0
    # holds the first four); every score in tile 0 equal -> the lowest slots
    rows = np.array([[1.0, 2.0]] * 4 + [[3.0, 1.0]])
    qt = _tiled(rows, (1, 1, 5))
    keep = prune.keep_mask(qt, 1, 1, 5, 0.5)
    assert list(np.nonzero(keep[0, 0, 0])[0]) == [0, 1]


@pytest.mark.parametrize("mode,tile", [("cumulative", (4, 4, 4)), ("topk", (4, 4, 4)),
                                       ("cumulative", (4, 4, 8)), ("topk", (4, 4, 8))])
def test_keep_all_is_the_unpruned_path(mode, tile):
    """ratio = 1 keeps every valid token: pooled, selection and output equal the
    unpruned path's, for 64-token and 128-token tiles."""
    w = workloads.custom("prune_all", 1, 2, 64, 5, 6, 11, "topk", 3, seed=64)
    inp = workloads.make_inputs(w)
    r = prune.run(inp["q"], inp["k"], inp["v"], w.T, w.Y, w.X, 1.0, mode=mode, threshold=0.6,
                  topk=w.topk, tile=tile)
    ref = pipeline.run(inp["q"], inp["k"], inp["v"], w.T, w.Y, w.X, "topk", w.topk, tile=tile)
    assert r["keep"].shape[3] == geometry.tile_elems(tile)
    assert np.array_equal(r["pq"], ref["pq"])
    if mode == "topk":
        assert np.array_equal(r["mask"], ref["mask"])
        assert np.array_equal(r["out"], ref["out"])
    else:
        D = w.D
        assert np.array_equal(r["mask"], select.cumulative_mask(ref["scores"], D, 0.6))


@pytest.mark.parametrize("tile", [(4, 4, 4), (4, 4, 8)])
def test_kept_rows_match_dense_brute_force_and_pruned_rows_are_zero(tile):
    """Kept rows equal a dense float64 brute force under the explicit token
    mask of the pruned path's own selection; pruned and pad rows are 0 with
    lse -inf; the selection is the cumulative rule on the kept queries' means;
    each tile keeps kept_count(n) tokens, those of lowest redundancy."""
    w = workloads.custom("prune_bf", 1, 2, 64, 6, 5, 9, "topk", 3, seed=65)
    inp = workloads.make_inputs(w)
    T, Y, X = w.T, w.Y, w.X
    E = geometry.tile_elems(tile)
    r = prune.run(inp["q"], inp["k"], inp["v"], T, Y, X, 0.4, mode="cumulative", threshold=0.5,
                  min_blocks=1, tile=tile)
    q, k, v = (workloads.bf16_to_f32(inp[n]).astype(np.float64) for n in ("q", "k", "v"))
    dense, dlse = attention.dense_masked_attention(q, k, v, r["mask"], T, Y, X, tile=tile)
    slots = geometry.token_slots(T, Y, X, tile)
    occ = geometry.occupancy(T, Y, X, tile)
    for h in range(w.H):
        for j, n in enumerate(occ):
            kept = np.nonzero(r["keep"][0, h, j])[0]
            assert len(kept) == prune.kept_count(int(n), 0.4) and kept.max() < n
            sc = prune.redundancy(r["qt"][0, j * E:j * E + n, h])
            assert sc[kept].max() <= np.delete(sc, kept).min() if len(kept) < n else True
    keep_tok = r["keep"].transpose(0, 2, 3, 1).reshape(1, -1, w.H)[:, slots]   # [B, L, H]
    assert keep_tok.sum() < keep_tok.size          # something was pruned
    assert np.allclose(r["out"][keep_tok], dense[keep_tok], rtol=0, atol=1e-10)
    assert np.all(r["out"][~keep_tok] == 0.0)
    lse_tok = r["lse"][:, :, slots]
    assert np.all(np.isneginf(lse_tok[~keep_tok.transpose(0, 2, 1)]))
    assert np.allclose(lse_tok[keep_tok.transpose(0, 2, 1)], dlse[keep_tok.transpose(0, 2, 1)],
                       rtol=0, atol=1e-10)
    # the selection is taken from the kept queries' means
    s = select.scores(r["pq"], r["pk"])
    assert np.array_equal(r["mask"], select.cumulative_mask(s, w.D, 0.5, 1))
    mean_kept = np.stack([[r["qt"][0, j * E + np.nonzero(r["keep"][0, h, j])[0], h].mean(axis=0)
                           for j in range(r["keep"].shape[2])] for h in range(w.H)])
    assert np.allclose(r["pq"][0], mean_kept, rtol=1e-6, atol=1e-6)
