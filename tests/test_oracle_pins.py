"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a closed form, a brute force built a
different way, a library routine on a special case, or a hand-derived fixture
in tests/golden.  A plausible slip in the oracle (a dropped term, a wrong
sign, index or operand order) fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import attention, geometry, pipeline, select, tiling

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- geometry

def test_occupancy_histogram_golden():
    g = _golden("geometry_examples.json")["occupancy_21x30x52"]
    T, Y, X = g["grid"]
    assert geometry.tile_counts(T, Y, X) == tuple(g["tile_counts"])
    occ = geometry.occupancy(T, Y, X)
    vals, counts = np.unique(occ, return_counts=True)
    assert {str(v): int(c) for v, c in zip(vals, counts)} == g["histogram"]
    assert occ.sum() == T * Y * X


@pytest.mark.parametrize("name", ["partition_2x3x5", "partition_5x4x4"])
def test_partition_golden(name):
    g = _golden("geometry_examples.json")[name]
    T, Y, X = g["grid"]
    assert list(geometry.occupancy(T, Y, X)) == g["occupancy"]
    if "tile_order" in g:
        assert list(geometry.tile_order(T, Y, X)) == g["tile_order"]
    if "slots_of_tokens_64_to_79" in g:
        assert list(geometry.token_slots(T, Y, X)[64:80]) == g["slots_of_tokens_64_to_79"]


@pytest.mark.parametrize("grid", [(8, 8, 8), (4, 12, 8), (16, 32, 32)])
def test_partition_divisible_equals_rearrange(grid):
    """Divisible grid: tile order = "(nt ts)(ny ys)(nx xs) -> (nt ny nx)(ts ys xs)"."""
    T, Y, X = grid
    ids = np.arange(T * Y * X).reshape(T // 4, 4, Y // 4, 4, X // 4, 4)
    expected = ids.transpose(0, 2, 4, 1, 3, 5).reshape(-1)
    assert np.array_equal(geometry.tile_order(T, Y, X), expected)
    assert np.array_equal(geometry.token_slots(T, Y, X), np.argsort(expected))


def _extent(dim, idx):
    """Tokens of tile idx along an axis of dim tokens cut into 4s."""
    return min(4, dim - 4 * idx)


@pytest.mark.parametrize("grid", [(5, 6, 7), (1, 1, 1), (3, 9, 2), (21, 30, 52), (4, 4, 5), (9, 13, 10)])
def test_occupancy_closed_form(grid):
    """n_j = s_t(a) s_y(b) s_x(c) with s(idx) = min(4, dim - 4 idx), tile j = (a nY + b) nX + c."""
    T, Y, X = grid
    nt, ny, nx = (math.ceil(T / 4), math.ceil(Y / 4), math.ceil(X / 4))
    occ = geometry.occupancy(T, Y, X)
    assert len(occ) == nt * ny * nx == geometry.num_tiles(T, Y, X)
    for a in range(nt):
        for b in range(ny):
            for c in range(nx):
                assert occ[(a * ny + b) * nx + c] == _extent(T, a) * _extent(Y, b) * _extent(X, c)
    assert occ.sum() == T * Y * X


@pytest.mark.parametrize("grid", [(5, 6, 7), (1, 1, 1), (3, 9, 2), (21, 30, 52), (4, 4, 5)])
def test_geometry_brute_force(grid):
    """Per-token tile id and rank by counting tokens in raster order."""
    T, Y, X = grid
    nt, ny, nx = (math.ceil(T / 4), math.ceil(Y / 4), math.ceil(X / 4))
    occ = geometry.occupancy(T, Y, X)
    slots = geometry.token_slots(T, Y, X)
    counts = np.zeros(nt * ny * nx, dtype=np.int64)
    seen = set()
    for l in range(T * Y * X):
        t, rem = divmod(l, Y * X)
        y, x = divmod(rem, X)
        j = ((t // 4) * ny + y // 4) * nx + x // 4
        r = counts[j]           # raster order inside a tile = rank so far
        counts[j] += 1
        assert slots[l] == 64 * j + r
        seen.add(int(slots[l]))
    assert np.array_equal(counts, occ)
    assert len(seen) == T * Y * X


@pytest.mark.parametrize("grid", [(5, 6, 7), (3, 9, 2), (21, 30, 52), (7, 5, 11)])
def test_slot_closed_form(grid):
    """slot = 64 j + (dt s_y(b) + dy) s_x(c) + dx with (dt, dy, dx) = (t, y, x) mod 4:
    the clipped sub-block's row-major rank, from the tile's own extents."""
    T, Y, X = grid
    ny, nx = math.ceil(Y / 4), math.ceil(X / 4)
    slots = geometry.token_slots(T, Y, X)
    order = geometry.tile_order(T, Y, X)
    for t in range(T):
        for y in range(Y):
            for x in range(X):
                a, b, c = t // 4, y // 4, x // 4
                r = ((t % 4) * _extent(Y, b) + y % 4) * _extent(X, c) + x % 4
                assert slots[(t * Y + y) * X + x] == 64 * ((a * ny + b) * nx + c) + r
    # the tile-contiguous order lists the tokens by increasing slot
    assert np.all(np.diff(slots[order]) > 0)


# ---------------------------------------------------------------- tiling

@pytest.mark.parametrize("grid", [(5, 6, 7), (8, 8, 8), (2, 3, 5)])
def test_tile_roundtrip_and_zero_pad(grid):
    T, Y, X = grid
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, T * Y * X, 3, 8)).astype(np.float32) + 10.0
    xt = tiling.tile(x, T, Y, X)
    assert xt.shape[1] == geometry.padded_len(T, Y, X)
    assert np.array_equal(tiling.untile(xt, T, Y, X), x)
    valid = np.zeros(xt.shape[1], dtype=bool)
    valid[geometry.token_slots(T, Y, X)] = True
    assert np.all(xt[:, ~valid] == 0.0)
    assert np.all(xt[:, valid] != 0.0)
    with pytest.raises(ValueError):
        tiling.tile(x[:, :-1], T, Y, X)


# ---------------------------------------------------------------- pooling

def test_pool_golden():
    g = _golden("select_examples.json")["pooled_example"]
    T, Y, X = g["grid"]
    q = np.array(g["q_rows"], dtype=np.float64)[None, :, None, :]
    k = np.array(g["k_rows"], dtype=np.float64)[None, :, None, :]
    pq = select.pool(tiling.tile(q, T, Y, X), T, Y, X)[0, 0]
    pk = select.pool(tiling.tile(k, T, Y, X), T, Y, X)[0, 0]
    assert np.array_equal(pq, np.array(g["pooled_q"], dtype=np.float32))
    assert np.array_equal(pk, np.array(g["pooled_k"], dtype=np.float32))
    s = select.scores(pq[None, None], pk[None, None])[0, 0]
    assert np.array_equal(s, np.array(g["scores"], dtype=np.float64))
    m = select.topk_mask(s, 1)
    assert [list(np.nonzero(r)[0]) for r in m] == g["top1"]


@pytest.mark.parametrize("grid", [(5, 6, 7), (8, 8, 8)])
def test_pool_matches_grouped_sum(grid):
    """Mean per tile from the raster input grouped by tile coordinates."""
    T, Y, X = grid
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, T * Y * X, 2, 5)).astype(np.float32)
    tid = geometry.token_tile_ids(T, Y, X)
    nt = tid.max() + 1
    sums = np.zeros((nt, 2, 5))
    np.add.at(sums, tid, x[0].astype(np.float64))
    cnt = np.bincount(tid)
    expected = (sums / cnt[:, None, None]).astype(np.float32).transpose(1, 0, 2)
    got = select.pool(tiling.tile(x, T, Y, X), T, Y, X)[0]
    assert np.array_equal(got, expected)


def test_pool_constant_tile():
    T, Y, X = 5, 6, 7
    x = np.full((1, T * Y * X, 1, 4), 0.3, dtype=np.float32)
    got = select.pool(tiling.tile(x, T, Y, X), T, Y, X)
    assert np.allclose(got, np.float32(0.3), rtol=0, atol=1e-7)


# ---------------------------------------------------------------- selection

def test_topk_golden_rows():
    for case in _golden("select_examples.json")["topk_rows"]:
        s = np.array([case["scores"]])
        m = select.topk_mask(s, case["k"])
        assert list(np.nonzero(m[0])[0]) == case["selected"], case


def _rank_select(row, k):
    """j kept iff fewer than k entries beat it (higher, or equal at a lower index)."""
    n = len(row)
    return np.array([sum(1 for jj in range(n) if row[jj] > row[j] or (row[jj] == row[j] and jj < j)) < k
                     for j in range(n)])


def test_topk_rank_definition_with_ties():
    rng = np.random.default_rng(11)
    for _ in range(200):
        n = int(rng.integers(1, 10))
        row = rng.integers(-3, 4, size=n).astype(np.float64) * 0.5   # many ties
        k = int(rng.integers(1, n + 1))
        assert np.array_equal(select.topk_mask(row[None], k)[0], _rank_select(row, k))


def test_topk_exhaustive_small():
    """Brute force over all k-subsets: the kept set is the unique one whose
    every member outranks every non-member."""
    rng = np.random.default_rng(5)
    for _ in range(40):
        n = 7
        row = rng.integers(-2, 3, size=n).astype(np.float64)
        for k in range(1, n + 1):
            winners = []
            for sub in itertools.combinations(range(n), k):
                inside = set(sub)
                ok = all(row[a] > row[b] or (row[a] == row[b] and a < b)
                         for a in inside for b in range(n) if b not in inside)
                if ok:
                    winners.append(sub)
            assert len(winners) == 1
            got = tuple(np.nonzero(select.topk_mask(row[None], k)[0])[0])
            assert got == winners[0]


def test_topk_zero_query_selects_first_k():
    """Q = 0 makes every score 0, so the tie rule keeps tiles 0..k-1."""
    T, Y, X = 8, 8, 8
    rng = np.random.default_rng(2)
    q = np.zeros((1, 512, 2, 16))
    k = rng.standard_normal((1, 512, 2, 16))
    res = pipeline.block_mask(tiling.tile(q, T, Y, X), tiling.tile(k, T, Y, X), T, Y, X, "topk", 3)
    assert np.all(res["scores"] == 0)
    assert np.all(res["mask"][..., :3]) and not np.any(res["mask"][..., 3:])


def test_scores_rank_one_orientation():
    """Pq rows = a_i u, Pk rows = b_j u  =>  S_ij = a_i b_j |u|^2 (not S^T)."""
    a = np.array([1.0, -2.0, 0.5])
    b = np.array([3.0, -1.0, 2.0, 0.25])
    u = np.array([1.0, 2.0, -2.0])
    pq = (a[:, None] * u[None])[None, None]
    pk = (b[:, None] * u[None])[None, None]
    s = select.scores(pq, pk)[0, 0]
    assert s.shape == (3, 4)
    assert np.allclose(s, np.outer(a, b) * 9.0, rtol=0, atol=1e-12)
    m = select.topk_mask(s, 1)
    assert [int(np.nonzero(r)[0][0]) for r in m] == [0, 1, 0]


def test_topk_all_tiles_and_counts():
    rng = np.random.default_rng(4)
    s = rng.standard_normal((2, 3, 9, 9))
    assert np.all(select.topk_mask(s, 9))
    m = select.topk_mask(s, 4)
    assert np.all(m.sum(-1) == 4)
    with pytest.raises(ValueError):
        select.topk_mask(s, 0)
    with pytest.raises(ValueError):
        select.topk_mask(s, 10)


def test_boundary_gap():
    s = np.array([[0.5, 2.0, 0.5, 1.0, 2.0]])
    assert select.boundary_gap(s, 2)[0] == 1.0
    assert select.boundary_gap(s, 1)[0] == 0.0
    assert select.boundary_gap(s, 5)[0] == np.inf
    up, lo = select.kth_values(s, 3)
    assert up[0] == 1.0 and lo[0] == 0.5


def test_cumulative_golden_rows():
    g = _golden("select_examples.json")["cumulative_rows"]
    for case in g["cases"]:
        s = np.array([case["scores"]])
        m = select.cumulative_mask(s, g["D"], case["threshold"], case["min_blocks"])
        assert list(np.nonzero(m[0])[0]) == case["selected"], case


def test_cumulative_masses_golden():
    """Prefix masses in descending score order at the attention's 1/sqrt(D),
    derived by hand (select_examples.json)."""
    g = _golden("select_examples.json")["cumulative_rows"]
    for case in g["prefix_masses"]:
        got = select.cumulative_masses(np.array([case["scores"]]), g["D"])[0]
        assert np.allclose(got, case["masses"], rtol=0, atol=1e-12), case


def _softmax_py(row, D):
    z = [v / math.sqrt(D) for v in row]
    top = max(z)
    e = [math.exp(v - top) for v in z]
    tot = math.fsum(e)
    return [v / tot for v in e]


def test_cumulative_brute_force_subsets():
    """The count is the least c for which SOME c-subset of tiles holds at
    least the threshold's mass (all subsets enumerated), raised to the
    minimum; the kept set is the c-subset of largest mass."""
    rng = np.random.default_rng(21)
    for _ in range(150):
        n = int(rng.integers(1, 8))
        D = int(rng.choice([16, 64, 128]))
        row = rng.standard_normal(n) * float(rng.choice([1.0, 8.0, 30.0]))
        tau = float(rng.uniform(0.01, 1.0))
        mb = int(rng.integers(0, n + 2))
        p = _softmax_py(row, D)
        best = {c: max(itertools.combinations(range(n), c), key=lambda sub: math.fsum(p[j] for j in sub))
                for c in range(1, n + 1)}
        c = next((c for c in range(1, n + 1) if math.fsum(p[j] for j in best[c]) >= tau), n)
        c = max(c, min(mb, n))
        got = select.cumulative_mask(row[None], D, tau, mb)[0]
        assert int(select.cumulative_counts(row[None], D, tau, mb)[0]) == c
        masses = select.cumulative_masses(row[None], D)[0]
        for cc in range(1, n + 1):
            assert abs(masses[cc - 1] - math.fsum(p[j] for j in best[cc])) < 1e-12
        assert tuple(np.nonzero(got)[0]) == tuple(sorted(best[c]))


def test_cumulative_small_threshold_is_topk():
    """A threshold below every tile's probability keeps max(1, min_blocks)
    tiles: the top-k selection with that k."""
    rng = np.random.default_rng(22)
    s = rng.integers(-3, 4, size=(3, 5, 40)).astype(np.float64)   # ties included
    for mb in (0, 1, 7, 40, 55):
        k = max(1, min(mb, 40))
        assert np.array_equal(select.cumulative_mask(s, 64, 1e-30, mb), select.topk_mask(s, k))


def test_cumulative_invariants():
    rng = np.random.default_rng(23)
    s = rng.standard_normal((4, 200)) * 20.0
    D = 128
    p = np.exp(s / math.sqrt(D) - (s / math.sqrt(D)).max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    prev = np.zeros(4, dtype=np.int64)
    for tau in (0.05, 0.2, 0.5, 0.8, 0.95, 1.0):
        m = select.cumulative_mask(s, D, tau)
        cnt = m.sum(-1)
        assert np.all(cnt >= prev)            # a higher threshold never keeps fewer
        prev = cnt
        kept = np.where(m, p, 0.0).sum(-1)
        assert np.all(kept >= tau - 1e-12)
        # dropping the weakest kept tile falls below the threshold
        weakest = np.where(m, p, np.inf).min(-1)
        assert np.all(kept - weakest < tau)
        # every kept tile outscores every dropped one
        assert np.all(np.where(m, s, np.inf).min(-1) >= np.where(m, -np.inf, s).max(-1))
    masses = select.cumulative_masses(s, D)
    assert np.allclose(masses[:, -1], 1.0, atol=1e-12)
    assert np.all(np.diff(masses, axis=-1) >= 0)


def test_cumulative_rejects_bad_arguments():
    s = np.zeros((1, 4))
    for tau in (0.0, -0.5, 1.5, float("nan")):
        with pytest.raises(ValueError):
            select.cumulative_counts(s, 64, tau)
    with pytest.raises(ValueError):
        select.cumulative_counts(s, 64, 0.5, -1)


def test_topk_from_ratio():
    assert select.topk_from_ratio(0.1, 1200) == 120
    assert select.topk_from_ratio(0.125, 256) == 32
    assert select.topk_from_ratio(2.0, 8) == 8


def test_sta_golden():
    g = _golden("select_examples.json")["sta_examples"]
    T, Y, X = g["grid"]
    nt, ny, nx = g["tile_counts"]
    for case in g["cases"]:
        m = select.sta_mask(T, Y, X, np.array([case["window"]]), 1)[0, 0]
        a, b, c = case["query_coords"]
        i = (a * ny + b) * nx + c
        exp = sorted((ta * ny + tb) * nx + tc for ta in case["key_coords_t"]
                     for tb in case["key_coords_y"] for tc in case["key_coords_x"])
        assert list(np.nonzero(m[i])[0]) == exp, case


@pytest.mark.parametrize("grid", [(16, 48, 80), (8, 12, 20), (5, 6, 7)])
def test_sta_invariants(grid):
    T, Y, X = grid
    n = geometry.tile_counts(T, Y, X)
    nt = n[0] * n[1] * n[2]
    full = select.sta_mask(T, Y, X, np.array([n]), 2)
    assert np.all(full)
    diag = select.sta_mask(T, Y, X, np.array([[1, 1, 1]]), 1)[0, 0]
    assert np.array_equal(diag, np.eye(nt, dtype=bool))
    wins = np.array([[min(w, n[0]), min(3, n[1]), min(5, n[2])] for w in (1, 3)])
    m = select.sta_mask(T, Y, X, wins, 1)[0]
    for h in range(2):
        assert np.all(m[h].sum(-1) == np.prod(wins[h]))
    with pytest.raises(ValueError):
        select.sta_mask(T, Y, X, np.array([[n[0] + 1, 1, 1]]), 1)


def test_sta_odd_window_centre_clamp():
    """Odd windows: centre c = clamp(a, w//2, n-1-w//2) and |a_j - c| <= w//2."""
    T, Y, X = 16, 48, 80
    n = geometry.tile_counts(T, Y, X)
    coords = geometry.tile_coords(T, Y, X)
    for win in [(1, 3, 3), (3, 3, 3), (3, 5, 5)]:
        m = select.sta_mask(T, Y, X, np.array([win]), 1)[0, 0]
        for i in range(0, len(coords), 37):
            keep = np.ones(len(coords), dtype=bool)
            for ax in range(3):
                r = win[ax] // 2
                c = min(max(coords[i, ax], r), n[ax] - 1 - r)
                keep &= np.abs(coords[:, ax] - c) <= r
            assert np.array_equal(m[i], keep)


def test_mask_to_csr():
    rng = np.random.default_rng(8)
    mask = rng.random((2, 3, 6, 6)) < 0.4
    rp, ci = select.mask_to_csr(mask)
    assert rp[0] == 0 and rp[-1] == mask.sum() and len(rp) == 2 * 3 * 6 + 1
    rows = mask.reshape(-1, 6)
    for r in range(len(rows)):
        cols = ci[rp[r]:rp[r + 1]]
        assert np.all(np.diff(cols) > 0)
        rebuilt = np.zeros(6, dtype=bool)
        rebuilt[cols] = True
        assert np.array_equal(rebuilt, rows[r])


# ---------------------------------------------------------------- attention

def test_attention_golden():
    g = _golden("attention_examples.json")
    T, Y, X = g["grid"]
    q = np.array(g["q"], dtype=np.float64)[None, :, None, :]
    k = np.array(g["k"], dtype=np.float64)[None, :, None, :]
    v = np.array(g["v"], dtype=np.float64)[None, :, None, :]
    mask = np.ones((1, 1, 1, 1), dtype=bool)
    out, lse = attention.block_sparse_attention(tiling.tile(q, T, Y, X), tiling.tile(k, T, Y, X),
                                                tiling.tile(v, T, Y, X), mask, T, Y, X)
    assert np.allclose(out[0, :2, 0], np.array(g["out"]), rtol=0, atol=1e-15)
    assert np.allclose(lse[0, 0, :2], np.array(g["lse"]), rtol=0, atol=1e-15)
    assert np.all(out[0, 2:] == 0) and np.all(np.isneginf(lse[0, 0, 2:]))


def _random_case(grid, H=2, D=16, B=1, seed=0):
    rng = np.random.default_rng(seed)
    L = grid[0] * grid[1] * grid[2]
    return [rng.standard_normal((B, L, H, D)) for _ in range(3)]


@pytest.mark.parametrize("grid,k", [((8, 8, 8), 2), ((5, 6, 7), 3), ((5, 6, 7), 1), ((3, 9, 2), 2)])
def test_attention_vs_dense_token_mask(grid, k):
    """Block-sparse attention == brute-force dense attention with a 0/-inf
    token mask built from the block mask, in raster order."""
    T, Y, X = grid
    q, kk, v = _random_case(grid, B=2)
    qt, kt, vt = (tiling.tile(a, T, Y, X) for a in (q, kk, v))
    res = pipeline.block_mask(qt, kt, T, Y, X, "topk", k)
    out_t, lse_t = attention.block_sparse_attention(qt, kt, vt, res["mask"], T, Y, X)
    dense, dlse = attention.dense_masked_attention(q, kk, v, res["mask"], T, Y, X)
    assert np.allclose(tiling.untile(out_t, T, Y, X), dense, rtol=0, atol=1e-12)
    slots = geometry.token_slots(T, Y, X)
    assert np.allclose(lse_t[:, :, slots], dlse, rtol=0, atol=1e-12)
    # padded query rows are exactly zero
    valid = np.zeros(out_t.shape[1], dtype=bool)
    valid[slots] = True
    assert np.all(out_t[:, ~valid] == 0)


@pytest.mark.parametrize("grid", [(8, 8, 8), (5, 6, 7)])
def test_all_tiles_equals_library_attention(grid):
    """k = Nt: untile(attn(tile(.))) is plain softmax attention (torch SDPA, float64)."""
    T, Y, X = grid
    q, kk, v = _random_case(grid, H=2, D=16)
    nt = geometry.num_tiles(T, Y, X)
    res = pipeline.run(*(pipeline_bits(a) for a in (q, kk, v)), T, Y, X, "topk", nt)
    qf, kf, vf = (pipeline.widen(pipeline_bits(a)) for a in (q, kk, v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(a).permute(0, 2, 1, 3) for a in (qf, kf, vf))).permute(0, 2, 1, 3).numpy()
    assert np.allclose(res["out"], ref, rtol=0, atol=1e-10)


def pipeline_bits(a):
    """float -> bf16 bits (truncation is fine here; both sides get the same bits)."""
    return (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_zero_query_gives_mean_of_selected_values():
    T, Y, X = 5, 6, 7
    _, kk, v = _random_case((T, Y, X), H=1, D=8, seed=9)
    q = np.zeros_like(kk)
    qt, kt, vt = (tiling.tile(a, T, Y, X) for a in (q, kk, v))
    rng = np.random.default_rng(1)
    nt = geometry.num_tiles(T, Y, X)
    mask = rng.random((1, 1, nt, nt)) < 0.5
    mask[..., 0] = True
    out, lse = attention.block_sparse_attention(qt, kt, vt, mask, T, Y, X)
    occ = geometry.occupancy(T, Y, X)
    for i in range(nt):
        sel = np.nonzero(mask[0, 0, i])[0]
        vals = np.concatenate([vt[0, j * 64:j * 64 + occ[j], 0] for j in sel])
        assert np.allclose(out[0, i * 64:i * 64 + occ[i], 0], vals.mean(0)[None], atol=1e-13)
        assert np.allclose(lse[0, 0, i * 64:i * 64 + occ[i]], math.log(len(vals)), atol=1e-13)


def test_constant_values_give_constant_output():
    T, Y, X = 5, 6, 7
    q, kk, _ = _random_case((T, Y, X), H=1, D=8, seed=3)
    v = np.full_like(q, -1.75)
    qt, kt, vt = (tiling.tile(a, T, Y, X) for a in (q, kk, v))
    res = pipeline.block_mask(qt, kt, T, Y, X, "topk", 2)
    out, _ = attention.block_sparse_attention(qt, kt, vt, res["mask"], T, Y, X)
    assert np.allclose(tiling.untile(out, T, Y, X), -1.75, atol=1e-13)


def test_single_tile_matches_textbook_and_logsumexp():
    """One selected tile: softmax over <= 64 keys, checked with torch and scipy."""
    T, Y, X = 5, 6, 7
    q, kk, v = _random_case((T, Y, X), H=1, D=8, seed=12)
    qt, kt, vt = (tiling.tile(a, T, Y, X) for a in (q, kk, v))
    nt = geometry.num_tiles(T, Y, X)
    mask = np.zeros((1, 1, nt, nt), dtype=bool)
    pick = [(i * 5 + 3) % nt for i in range(nt)]
    for i, j in enumerate(pick):
        mask[0, 0, i, j] = True
    out, lse = attention.block_sparse_attention(qt, kt, vt, mask, T, Y, X)
    occ = geometry.occupancy(T, Y, X)
    for i, j in enumerate(pick):
        qi = torch.from_numpy(qt[0, i * 64:i * 64 + occ[i], 0])
        kj = torch.from_numpy(kt[0, j * 64:j * 64 + occ[j], 0])
        vj = torch.from_numpy(vt[0, j * 64:j * 64 + occ[j], 0])
        ref = torch.nn.functional.scaled_dot_product_attention(qi[None], kj[None], vj[None])[0].numpy()
        assert np.allclose(out[0, i * 64:i * 64 + occ[i], 0], ref, atol=1e-12)
        s = (qi.numpy() @ kj.numpy().T) / math.sqrt(8)
        assert np.allclose(lse[0, 0, i * 64:i * 64 + occ[i]], logsumexp(s, axis=1), atol=1e-12)


# ---------------------------------------------------------------- backward

def _bwd_case(grid, H=2, D=16, B=1, k=3, seed=0, tile=geometry.TILE):
    T, Y, X = grid
    rng = np.random.default_rng(seed)
    L = T * Y * X
    q, kk, v, do = (rng.standard_normal((B, L, H, D)) for _ in range(4))
    nt = geometry.num_tiles(T, Y, X, tile)
    s = rng.standard_normal((B, H, nt, nt))
    mask = select.topk_mask(s, min(k, nt))
    return q, kk, v, do, mask


@pytest.mark.parametrize("grid,k,tile", [((5, 6, 7), 2, (4, 4, 4)), ((8, 8, 4), 3, (4, 4, 4)),
                                         ((3, 9, 5), 1, (4, 4, 4)), ((5, 6, 11), 2, (4, 4, 8)),
                                         ((4, 8, 16), 3, (4, 4, 8))])
def test_backward_equals_autograd(grid, k, tile):
    """torch autograd (float64) through the dense token-masked attention, for
    64-token and 128-token tiles (the token mask comes from each token's tile
    coordinates, not from the slot order the oracle walks)."""
    T, Y, X = grid
    q, kk, v, do, mask = _bwd_case(grid, k=k, seed=7, tile=tile)
    B, L, H, D = q.shape
    tid = geometry.token_tile_ids(T, Y, X, tile)
    qt_, kt_, vt_ = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, kk, v))
    out = torch.zeros((B, L, H, D), dtype=torch.float64)
    outs = []
    for b in range(B):
        for h in range(H):
            tokmask = torch.tensor(np.where(mask[b, h][tid][:, tid], 0.0, -np.inf))
            sc = qt_[b, :, h] @ kt_[b, :, h].T / math.sqrt(D) + tokmask
            outs.append(torch.softmax(sc, dim=-1) @ vt_[b, :, h])
    out = torch.stack(outs).reshape(B, H, L, D).permute(0, 2, 1, 3)
    (out * torch.tensor(do)).sum().backward()
    tq, tk, tv, tdo = (tiling.tile(a, T, Y, X, tile) for a in (q, kk, v, do))
    dq, dk, dv = attention.block_sparse_attention_backward(tq, tk, tv, tdo, mask, T, Y, X, tile=tile)
    for got, ref in ((dq, qt_.grad), (dk, kt_.grad), (dv, vt_.grad)):
        assert np.allclose(tiling.untile(got, T, Y, X, tile), ref.numpy(), rtol=1e-10, atol=1e-10)
    # pad slots receive nothing
    valid = np.zeros(tq.shape[1], dtype=bool)
    valid[geometry.token_slots(T, Y, X, tile)] = True
    for g in (dq, dk, dv):
        assert np.all(g[:, ~valid] == 0)


def test_backward_finite_differences():
    """Central differences of sum(dO * O) from the oracle's forward."""
    grid = (5, 4, 6)
    T, Y, X = grid
    q, kk, v, do, mask = _bwd_case(grid, D=8, k=2, seed=9)
    tq, tk, tv, tdo = (tiling.tile(a, T, Y, X) for a in (q, kk, v, do))
    grads = attention.block_sparse_attention_backward(tq, tk, tv, tdo, mask, T, Y, X)
    slots = geometry.token_slots(T, Y, X)
    rng = np.random.default_rng(3)

    def loss(a, b_, c):
        return float((attention.block_sparse_attention(a, b_, c, mask, T, Y, X)[0] * tdo).sum())

    eps = 1e-6
    for which in range(3):
        for _ in range(6):
            slot = int(rng.choice(slots))
            h, d = int(rng.integers(2)), int(rng.integers(8))
            args = [tq.copy(), tk.copy(), tv.copy()]
            args[which][0, slot, h, d] += eps
            up = loss(*args)
            args[which][0, slot, h, d] -= 2 * eps
            dn = loss(*args)
            fd = (up - dn) / (2 * eps)
            assert abs(fd - grads[which][0, slot, h, d]) <= 1e-6 * (1 + abs(fd)), (which, slot, h, d)


def test_backward_closed_forms():
    grid = (4, 8, 8)
    T, Y, X = grid
    q, kk, v, do, mask = _bwd_case(grid, k=3, seed=5)
    tq, tk, tv, tdo = (tiling.tile(a, T, Y, X) for a in (q, kk, v, do))
    # dO = 0: no gradient anywhere.
    z = attention.block_sparse_attention_backward(tq, tk, tv, np.zeros_like(tdo), mask, T, Y, X)
    assert all(np.all(g == 0) for g in z)
    # Equal value rows make the output independent of the scores: dQ = dK = 0,
    # and every query's dO is shared out over its keys with weights summing
    # to one, so dV sums (over keys) to dO summed over the queries.
    vc = np.broadcast_to(np.arange(16.0), tv.shape).copy()
    dq, dk, dv = attention.block_sparse_attention_backward(tq, tk, vc, tdo, mask, T, Y, X)
    assert np.allclose(dq, 0, atol=1e-12) and np.allclose(dk, 0, atol=1e-12)
    assert np.allclose(dv.sum(axis=1), _dv_total(tdo, mask, T, Y, X), atol=1e-9)


def _dv_total(tdo, mask, T, Y, X):
    """Sum over queries of dO, each query tile counted once per (row with a
    non-empty selection): [B, H, D]."""
    E = geometry.TILE_ELEMS
    occ = geometry.occupancy(T, Y, X)
    B, _, H, D = tdo.shape
    tot = np.zeros((B, H, D))
    for b in range(B):
        for h in range(H):
            for i in range(len(occ)):
                if mask[b, h, i].any():
                    tot[b, h] += tdo[b, i * E:i * E + occ[i], h].sum(axis=0)
    return tot


def test_sta_full_window_equals_dense():
    T, Y, X = 8, 8, 12
    q, kk, v = _random_case((T, Y, X), H=2, D=8, B=2, seed=6)
    n = geometry.tile_counts(T, Y, X)
    bits = [pipeline_bits(a) for a in (q, kk, v)]
    res = pipeline.run(*bits, T, Y, X, "sta", windows=np.array([n, n]))
    qf, kf, vf = (pipeline.widen(b) for b in bits)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(a).permute(0, 2, 1, 3) for a in (qf, kf, vf))).permute(0, 2, 1, 3).numpy()
    assert np.allclose(res["out"], ref, rtol=0, atol=1e-10)


# ---------------------------------------------------------------- 128-token tiles

T448 = geometry.TILE_SHAPES[128]


def test_tile128_partition_golden():
    g = _golden("geometry_examples.json")["partition_2x3x10_tile448"]
    assert tuple(g["tile"]) == T448
    T, Y, X = g["grid"]
    assert list(geometry.tile_order(T, Y, X, T448)) == g["tile_order"]
    assert list(geometry.occupancy(T, Y, X, T448)) == g["occupancy"]
    assert geometry.padded_len(T, Y, X, T448) == 2 * 128


def test_tile128_occupancy_histogram_golden():
    g = _golden("geometry_examples.json")["occupancy_21x30x52_tile448"]
    T, Y, X = g["grid"]
    assert geometry.tile_counts(T, Y, X, T448) == tuple(g["tile_counts"])
    vals, counts = np.unique(geometry.occupancy(T, Y, X, T448), return_counts=True)
    assert {str(v): int(c) for v, c in zip(vals, counts)} == g["histogram"]


@pytest.mark.parametrize("grid", [(8, 8, 16), (4, 12, 24)])
def test_tile128_divisible_equals_rearrange(grid):
    """Divisible grid: "(nt 4)(ny 4)(nx 8) -> (nt ny nx)(4 4 8)"."""
    T, Y, X = grid
    ids = np.arange(T * Y * X).reshape(T // 4, 4, Y // 4, 4, X // 8, 8)
    expected = ids.transpose(0, 2, 4, 1, 3, 5).reshape(-1)
    assert np.array_equal(geometry.tile_order(T, Y, X, T448), expected)
    assert np.array_equal(geometry.token_slots(T, Y, X, T448), np.argsort(expected))


@pytest.mark.parametrize("grid", [(5, 6, 7), (3, 9, 19), (1, 1, 1), (6, 5, 17)])
def test_tile128_brute_force_and_closed_forms(grid):
    """Tile id and rank by counting in raster order; occupancy and slot from
    the per-axis extents min(4, .), min(4, .), min(8, .)."""
    T, Y, X = grid
    ny, nx = math.ceil(Y / 4), math.ceil(X / 8)
    slots = geometry.token_slots(T, Y, X, T448)
    occ = geometry.occupancy(T, Y, X, T448)
    counts = np.zeros(len(occ), dtype=np.int64)
    for l in range(T * Y * X):
        t, rem = divmod(l, Y * X)
        y, x = divmod(rem, X)
        a, b, c = t // 4, y // 4, x // 8
        j = (a * ny + b) * nx + c
        sy, sx = min(4, Y - 4 * b), min(8, X - 8 * c)
        assert slots[l] == 128 * j + counts[j]
        assert slots[l] == 128 * j + ((t % 4) * sy + y % 4) * sx + x % 8
        counts[j] += 1
    assert np.array_equal(counts, occ)
    for j in range(len(occ)):
        a, rest = divmod(j, ny * nx)
        b, c = divmod(rest, nx)
        assert occ[j] == min(4, T - 4 * a) * min(4, Y - 4 * b) * min(8, X - 8 * c)


def test_tile128_pool_and_attention_brute_force():
    """128-token tiles through pooling (grouped float64 sums), top-k and the
    attention, against a dense float64 brute force with the explicit token
    mask; all tiles selected equals plain softmax attention."""
    rng = np.random.default_rng(81)
    T, Y, X = 5, 6, 19
    B, Hh, D = 1, 2, 16
    L = T * Y * X
    q, k, v = (rng.standard_normal((B, L, Hh, D)) for _ in range(3))
    qt, kt, vt = (tiling.tile(x, T, Y, X, T448) for x in (q, k, v))
    assert np.array_equal(tiling.untile(qt, T, Y, X, T448), q)
    tid = geometry.token_tile_ids(T, Y, X, T448)
    nt = geometry.num_tiles(T, Y, X, T448)
    sums = np.zeros((nt, Hh, D))
    np.add.at(sums, tid, q[0])
    want = (sums / np.bincount(tid)[:, None, None]).astype(np.float32).transpose(1, 0, 2)
    pq = select.pool(qt, T, Y, X, T448)
    assert np.array_equal(pq[0], want)
    s = select.scores(pq, select.pool(kt, T, Y, X, T448))
    mask = select.topk_mask(s, 2)
    out_t, lse_t = attention.block_sparse_attention(qt, kt, vt, mask, T, Y, X, tile=T448)
    dense, dlse = attention.dense_masked_attention(q, k, v, mask, T, Y, X, tile=T448)
    slots = geometry.token_slots(T, Y, X, T448)
    assert np.allclose(out_t[:, slots], dense, rtol=0, atol=1e-12)
    assert np.allclose(lse_t[:, :, slots], dlse, rtol=0, atol=1e-12)
    full = np.ones((B, Hh, nt, nt), dtype=bool)
    out_f, _ = attention.block_sparse_attention(qt, kt, vt, full, T, Y, X, tile=T448)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.transpose(0, 2, 1, 3)), torch.from_numpy(k.transpose(0, 2, 1, 3)),
        torch.from_numpy(v.transpose(0, 2, 1, 3))).numpy().transpose(0, 2, 1, 3)
    assert np.allclose(tiling.untile(out_f, T, Y, X, T448), ref, rtol=0, atol=1e-10)
