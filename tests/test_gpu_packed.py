"""GPU parity of packed multi-region sequences (reading R24) against
oracle/packed.py: dense prefix segments, reference video regions at
ref_keep_rate, the generated region at 1 - sparsity, exempt and compete
selection, patch division.

Bars as for a single grid: tile/untile bit-exact, pooled vectors within
1e-5(1+|x|), every selection row exact outside the 1e-4 tie band (prefix
rows and prefix columns exact), attention within max-abs 2e-2 / mean-abs
2e-3 (lse 5e-3), pad rows +0.0.
"""
import math

import numpy as np
import pytest

import workloads
from oracle import packed, select
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

CASES = {
    # name: (B, H, D, packed segments, patch, sparsity, ref_keep_rate, exempt, structure, seed)
    "ragged_two_regions": (1, 2, 64, [5, (1, 2, 5), 3, (2, 2, 2)], (1, 1, 1), 0.5, 0.5, True,
                           "none", 301),
    "d128_long_prefix": (2, 3, 128, [7, (1, 4, 6), 70, (4, 4, 5)], (1, 1, 1), 0.6, 0.5, True,
                         "none", 302),
    "patch_one_region": (1, 2, 128, [0, (8, 16, 24), 130], (1, 2, 2), 0.75, None, True, "smooth", 303),
    "compete": (1, 4, 128, [100, (8, 12, 16)], (1, 1, 1), 0.75, None, False, "smooth", 304),
    "three_regions": (1, 4, 128, [226, (8, 16, 20), (6, 16, 20), (12, 16, 20)], (1, 1, 1), 0.8, 0.3,
                      True, "smooth", 305),
    "dense_build": (1, 2, 64, [33, (5, 6, 7), (4, 4, 9)], (1, 1, 1), 0.0, 0.5, True, "none", 306),
    # the most segments: eight dense (one empty, dropped) and eight regions, one of a single token
    "sixteen_segments": (1, 2, 64, [3, (1, 2, 3), 70, (2, 4, 4), 1, (4, 4, 4), 65, (1, 1, 1), 0,
                                    (3, 5, 2), 128, (2, 2, 9), 5, (4, 8, 4), 7, (1, 3, 3)],
                         (1, 1, 1), 0.5, 0.4, True, "none", 310),
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


def _setup(case):
    B, Hh, D, segs, patch, sparsity, ref, exempt, structure, seed = case
    tsegs = packed.token_segments(segs, patch)
    lay = packed.layout(tsegs)
    inp = workloads.make_packed_inputs(B, Hh, D, tsegs, seed, structure)
    return dict(B=B, H=Hh, D=D, segs=segs, patch=patch, sparsity=sparsity, ref=ref, exempt=exempt,
                lay=lay, inp=inp)


def _run(m, c, fused=False):
    import torch
    g = m.Geometry.packed(c["B"], c["H"], c["D"], c["segs"], c["patch"])
    q, k, v = (H.to_dev(c["inp"][n]) for n in ("q", "k", "v"))
    if fused:
        nt = g.num_tiles
        ws = torch.empty(m.attn_workspace_bytes(g, m.SELECT_TOPK) // 4, dtype=torch.float32,
                         device="cuda")
        cap = m.attn_packed_capacity(g, c["sparsity"], c["ref"], c["exempt"])
        sel = m.Selection(torch.empty(c["B"] * c["H"] * nt + 1, dtype=torch.int32, device="cuda"),
                          torch.empty(cap, dtype=torch.int32, device="cuda"),
                          torch.empty((c["B"], c["H"], nt, nt), dtype=torch.uint8, device="cuda"), ws)
        pq, pk = sel.pooled(g)
        qt, kt = m.attn_tile_pool(g, q, pq), m.attn_tile_pool(g, k, pk)
        m.attn_select_packed(g, None, None, c["sparsity"], c["ref"], c["exempt"], prepooled=True,
                             out=sel)
    else:
        qt, kt = m.attn_tile(g, q), m.attn_tile(g, k)
        sel = m.attn_select_packed(g, qt, kt, c["sparsity"], c["ref"], c["exempt"])
    vt = m.attn_tile(g, v)
    ot, lse = m.attn_block_sparse_fwd(g, qt, kt, vt, sel.row_ptr, sel.col_idx, want_lse=True)
    o = torch.full((c["B"], g.L, c["H"], c["D"]), float("nan"), dtype=torch.bfloat16, device="cuda")
    m.attn_block_sparse_fwd(g, qt, kt, vt, sel.row_ptr, sel.col_idx, out=o, raster=True)
    torch.cuda.synchronize()
    return dict(g=g, qt=qt, kt=kt, vt=vt, sel=sel, ot=ot, lse=lse, o=o)


def _accept_selection(c, gmask, scores):
    """Prefix rows and prefix columns exact; each span (exempt) or each whole
    row (compete) a top-k row under the tie band."""
    lay = c["lay"]
    P = lay["num_prefix"]
    nt = len(lay["occ"])
    if not c["exempt"]:
        k = nt if c["sparsity"] <= 0 else packed.keep_count(nt, 1.0 - c["sparsity"])
        return H.accept_topk_rows(gmask, scores, k)
    assert gmask[:, :, :P].all(), "prefix query tiles keep every tile"
    assert gmask[:, :, P:, :P].all(), "video query tiles keep the whole prefix"
    keeps = packed.span_keeps(lay, c["sparsity"], c["ref"])
    exact = band = 0
    for (a, b), keep in zip(lay["spans"], keeps):
        k = packed.keep_count(b - a, keep)
        e, bd = H.accept_topk_rows(np.ascontiguousarray(gmask[:, :, P:, a:b]),
                                   np.ascontiguousarray(scores[:, :, P:, a:b]), k)
        exact, band = exact + e, band + bd
    return exact, band


def _check_path(m, c, r):
    lay = c["lay"]
    inp = c["inp"]
    tb = {n: packed.tile(inp[n], lay) for n in ("q", "k", "v")}
    for n in ("q", "k", "v"):
        assert np.array_equal(H.from_dev(r[n + "t"]), tb[n]), f"tiled {n}"
    assert np.array_equal(H.from_dev(m.attn_untile(r["g"], r["qt"])), inp["q"])
    tf = {n: workloads.bf16_to_f32(tb[n]) for n in tb}
    pq, pk = packed.pool(tf["q"], lay), packed.pool(tf["k"], lay)
    gpq, gpk = (t.cpu().numpy() for t in r["sel"].pooled(r["g"]))
    assert np.all(np.abs(gpq - pq) <= H.POOL_TOL * (1 + np.abs(pq)))
    assert np.all(np.abs(gpk - pk) <= H.POOL_TOL * (1 + np.abs(pk)))
    scores = np.matmul(pq.astype(np.float64), np.swapaxes(pk.astype(np.float64), -1, -2))
    gmask = r["sel"].block_mask.cpu().numpy().astype(bool)
    exact, band = _accept_selection(c, gmask, scores)
    H.log(f"  selection rows exact {exact}, inside tie band {band}")
    rp, ci = select.mask_to_csr(gmask)
    assert np.array_equal(r["sel"].row_ptr.cpu().numpy(), rp)
    assert np.array_equal(r["sel"].col_idx.cpu().numpy()[:len(ci)], ci)
    assert len(ci) == r["sel"].col_idx.numel(), "capacity equals the entries written"
    ref, rlse = packed.attention(tf["q"], tf["k"], tf["v"], gmask, lay)
    valid = lay["slot_token"] >= 0
    H.compare_outputs(H.bf16_dev_to_f32(r["ot"])[:, valid], ref[:, valid], "tiled output")
    assert np.all(H.from_dev(r["ot"])[:, ~valid] == 0), "pad rows +0.0"
    lse = r["lse"].cpu().numpy()
    assert np.all(np.isneginf(lse[:, :, ~valid]))
    assert np.abs(lse[:, :, valid] - rlse[:, :, valid]).max() <= H.LSE_TOL
    raster = H.bf16_dev_to_f32(r["o"])
    assert not np.isnan(raster).any(), "every raster row is written"
    H.compare_outputs(raster, packed.untile(ref, lay), "raster output")
    return gmask


@pytest.mark.parametrize("name", sorted(CASES))
def test_packed_path(bsta, name):
    """Tiling, pooling, the packed selection and the attention against the
    oracle (attention under the GPU's validated selection)."""
    c = _setup(CASES[name])
    H.log(f"packed {name}: Nt {len(c['lay']['occ'])}, prefix {c['lay']['num_prefix']}, "
          f"spans {c['lay']['spans']}")
    r = _run(bsta, c)
    gmask = _check_path(bsta, c, r)
    if c["sparsity"] <= 0:
        assert gmask.all(), "sparsity 0 keeps every tile"


@pytest.mark.parametrize("name", ["three_regions", "compete"])
def test_packed_fused_tile_pool(bsta, name):
    """attn_tile_pool + a prepooled packed selection: the same tiles, pooled
    vectors bit for bit, and the same CSR as the unfused route (the
    attention outputs may differ in rounding: each call starts its key walk
    at its own rotation)."""
    import torch
    c = _setup(CASES[name])
    a = _run(bsta, c)
    b = _run(bsta, c, fused=True)
    assert torch.equal(a["qt"].view(torch.int16), b["qt"].view(torch.int16))
    for x, y in zip(a["sel"].pooled(a["g"]), b["sel"].pooled(b["g"])):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    assert torch.equal(a["sel"].row_ptr, b["sel"].row_ptr)
    assert torch.equal(a["sel"].col_idx, b["sel"].col_idx)


def test_packed_dense_is_full_attention(bsta):
    """Sparsity 0: the GPU output equals plain softmax attention over the
    whole packed sequence (float64 on the CPU)."""
    c = _setup(CASES["dense_build"])
    r = _run(bsta, c)
    q, k, v = (workloads.bf16_to_f32(c["inp"][n]).astype(np.float64) for n in ("q", "k", "v"))
    s = np.einsum("blhd,bmhd->bhlm", q, k) / math.sqrt(c["D"])
    p = np.exp(s - s.max(-1, keepdims=True))
    ref = np.einsum("bhlm,bmhd->blhd", p / p.sum(-1, keepdims=True), v)
    H.compare_outputs(H.bf16_dev_to_f32(r["o"]), ref, "dense packed vs full attention")


@pytest.mark.parametrize("name", ["ragged_two_regions", "three_regions"])
def test_packed_backward(bsta, name):
    """attn_block_sparse_bwd on a packed geometry: dQ, dK, dV against the
    packed oracle under the per-element bound of the single-grid backward
    tests; pad slots +0.0."""
    import torch
    c = _setup(CASES[name])
    lay = c["lay"]
    r = _run(bsta, c)
    g = r["g"]
    rng = np.random.default_rng(309)
    do_bits = workloads.bf16_bits(rng.standard_normal((c["B"], g.L, c["H"], c["D"])).astype(np.float32))
    dot = bsta.attn_tile(g, H.to_dev(do_bits))
    grads = bsta.attn_block_sparse_bwd(g, r["qt"], r["kt"], r["vt"], r["ot"], dot, r["lse"],
                                       r["sel"].row_ptr, r["sel"].col_idx)
    torch.cuda.synchronize()
    mask = r["sel"].block_mask.cpu().numpy().astype(bool)
    tf = {n: workloads.bf16_to_f32(packed.tile(c["inp"][n], lay)) for n in ("q", "k", "v")}
    dtf = workloads.bf16_to_f32(packed.tile(do_bits, lay))
    ref = packed.attention_backward(tf["q"], tf["k"], tf["v"], dtf, mask, lay)
    bnd = H.backward_error_bounds(tf["q"], tf["k"], tf["v"], dtf, mask, 0, 0, 0, occ=lay["occ"])
    valid = lay["slot_token"] >= 0
    for nm, gt, rf, bd in zip(("dq", "dk", "dv"), grads, ref, bnd):
        bits = H.from_dev(gt)
        got = workloads.bf16_to_f32(bits).astype(np.float64)
        err = np.abs(got[:, valid] - rf[:, valid])
        ratio = float((err / (bd[:, valid] + 1e-6)).max())
        H.log(f"  {nm}: max err {err.max():.3g}, max err/bound {ratio:.3f}")
        assert np.all(err <= bd[:, valid] + 1e-6), f"{nm}: error above its bound (ratio {ratio:.3f})"
        assert np.all(bits[:, ~valid] == 0), f"{nm}: pad slots must be +0.0"


@pytest.mark.timeout(900)
def test_packed_full_size(bsta):
    """A 226-row dense prefix, a 4x48x80 reference region at keep 0.5 and the
    20x48x80 generated region at sparsity 0.9, 40 heads of 128: 1444 tiles.
    Tiles bit-exact, every selection row under the tie band, and one query
    tile per head against the oracle."""
    segs = [226, (4, 48, 80), (20, 48, 80)]
    c = dict(B=1, H=40, D=128, segs=segs, patch=(1, 1, 1), sparsity=0.9, ref=0.5, exempt=True)
    c["lay"] = lay = packed.layout(packed.token_segments(segs))
    H.log("packed full size: inputs")
    c["inp"] = inp = workloads.make_packed_inputs(1, 40, 128, packed.token_segments(segs), 307,
                                                  "smooth")
    r = _run(bsta, c, fused=True)
    tb = {n: packed.tile(inp[n], lay) for n in ("q", "k")}
    assert np.array_equal(H.from_dev(r["qt"]), tb["q"])
    tf = {n: workloads.bf16_to_f32(tb[n]) for n in tb}
    pq, pk = packed.pool(tf["q"], lay), packed.pool(tf["k"], lay)
    del tf
    gpq = r["sel"].pooled(r["g"])[0].cpu().numpy()
    assert np.all(np.abs(gpq - pq) <= H.POOL_TOL * (1 + np.abs(pq)))
    scores = np.matmul(pq.astype(np.float64), np.swapaxes(pk.astype(np.float64), -1, -2))
    gmask = r["sel"].block_mask.cpu().numpy().astype(bool)
    exact, band = _accept_selection(c, gmask, scores)
    H.log(f"  rows exact {exact}, inside tie band {band}")
    del scores
    nt = len(lay["occ"])
    rng = np.random.default_rng(308)
    rows = [(0, h, int(rng.integers(nt))) for h in range(40)]
    rows[0] = (0, 0, 0)                       # a prefix query tile (attends everything)
    rows[1] = (0, 1, nt - 1)                  # the last generated tile
    tf = {n: workloads.bf16_to_f32(packed.tile(inp[n], lay)) for n in ("q", "k", "v")}
    ref, _ = packed.attention(tf["q"], tf["k"], tf["v"], gmask, lay, rows=rows)
    got = H.bf16_dev_to_f32(r["o"])
    st = lay["slot_token"]
    gs, rs = [], []
    for b, h, i in rows:
        n = lay["occ"][i]
        gs.append(got[b, st[i * 64:i * 64 + n], h])
        rs.append(ref[b, i * 64:i * 64 + n, h])
    mx, mean = H.compare_outputs(np.concatenate(gs), np.concatenate(rs), "raster rows")
    H.log(f"  raster rows max-abs {mx:.3g}, mean-abs {mean:.3g}")
