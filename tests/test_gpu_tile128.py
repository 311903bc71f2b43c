"""GPU parity of the 128-token (4x4x8) tile variant against the CPU oracle run
with the same tile shape (reading R23).

Bars as for 64-token tiles: tile/untile and window masks bit-exact, top-k
rows exact outside the 1e-4 tie band, pooled vectors within 1e-5(1+|x|),
attention within max-abs 2e-2 / mean-abs 2e-3 (lse 5e-3), pad rows +0.0;
gradients within the per-element bound of tests/gpu_helpers.py
(backward_error_bounds), pad slots +0.0.
"""
import numpy as np
import pytest

import workloads
from oracle import attention as oatt
from oracle import geometry, pipeline, select, tiling
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

T448 = geometry.TILE_SHAPES[128]
CASES = {
    "ragged_d128": workloads.custom("t128_ragged_d128", 2, 3, 128, 5, 6, 19, "topk", 2, seed=91),
    "ragged_d64": workloads.custom("t128_ragged_d64", 1, 2, 64, 9, 13, 10, "topk", 3, seed=92),
    "smooth": workloads.custom("t128_smooth", 1, 4, 128, 8, 16, 24, "topk", 5, "smooth", seed=93),
    "one_token": workloads.custom("t128_one_token", 1, 1, 128, 1, 1, 1, "topk", 1, seed=94),
    "all_tiles": workloads.custom("t128_all_tiles", 1, 2, 128, 6, 7, 17, "topk", 12, seed=95),
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


def _geom(m, w):
    return m.Geometry(w.B, w.H, w.D, w.T, w.Y, w.X, tile_x=8)


def _oracle_tiled(w, inp):
    tb = {n: tiling.tile(inp[n], w.T, w.Y, w.X, T448) for n in ("q", "k", "v")}
    return tb, {n: workloads.bf16_to_f32(tb[n]) for n in tb}


def _run(m, w, inp, windows=None, fused=False):
    import torch
    g = _geom(m, w)
    q, k, v = (H.to_dev(inp[n]) for n in ("q", "k", "v"))
    mode = m.SELECT_STA if windows is not None else m.SELECT_TOPK
    if fused:
        sel = m.attn_select_alloc(g, mode, w.topk, windows)
        pq, pk = sel.pooled(g)
        qt, kt = m.attn_tile_pool(g, q, pq), m.attn_tile_pool(g, k, pk)
        vt = m.attn_tile(g, v)
        m.attn_select_blocks(g, None, None, mode | m.SELECT_PREPOOLED, w.topk, out=sel)
    else:
        qt, kt, vt = m.attn_tile(g, q), m.attn_tile(g, k), m.attn_tile(g, v)
        sel = m.attn_select_blocks(g, qt, kt, mode, w.topk, windows)
    ot, lse = m.attn_block_sparse_fwd(g, qt, kt, vt, sel.row_ptr, sel.col_idx, want_lse=True)
    o = torch.full((w.B, w.L, w.H, w.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    m.attn_block_sparse_fwd(g, qt, kt, vt, sel.row_ptr, sel.col_idx, out=o, raster=True)
    torch.cuda.synchronize()
    return dict(g=g, qt=qt, kt=kt, vt=vt, sel=sel, ot=ot, lse=lse, o=o)


def _check_outputs(w, r, ref_t, ref_lse):
    valid = np.zeros(ref_t.shape[1], dtype=bool)
    valid[geometry.token_slots(w.T, w.Y, w.X, T448)] = True
    got = H.bf16_dev_to_f32(r["ot"])
    H.compare_outputs(got[:, valid], ref_t[:, valid], "tiled output")
    assert np.all(H.from_dev(r["ot"])[:, ~valid] == 0), "pad rows +0.0"
    lse = r["lse"].cpu().numpy()
    assert np.all(np.isneginf(lse[:, :, ~valid]))
    assert np.abs(lse[:, :, valid] - ref_lse[:, :, valid]).max() <= H.LSE_TOL
    raster = H.bf16_dev_to_f32(r["o"])
    assert not np.isnan(raster).any(), "every raster row is written"
    H.compare_outputs(raster, tiling.untile(ref_t, w.T, w.Y, w.X, T448), "raster output")


@pytest.mark.parametrize("name", sorted(CASES))
def test_tile128_path(bsta, name):
    """Tiling bit-exact (and untile of it the identity), pooled vectors, the
    top-k selection under the tie band, and the attention (tiled and raster
    outputs, lse) against the oracle under the GPU's validated selection."""
    w = CASES[name]
    inp = H.inputs(w)
    H.log(f"128-token tiles {name}")
    r = _run(bsta, w, inp)
    tb, tf = _oracle_tiled(w, inp)
    for n in ("q", "k", "v"):
        assert np.array_equal(H.from_dev(r[n + "t"]), tb[n]), f"tiled {n}"
    assert np.array_equal(H.from_dev(bsta.attn_untile(r["g"], r["qt"])), inp["q"])
    pq = select.pool(tf["q"], w.T, w.Y, w.X, T448)
    pk = select.pool(tf["k"], w.T, w.Y, w.X, T448)
    gpq, gpk = (t.cpu().numpy() for t in r["sel"].pooled(r["g"]))
    assert np.all(np.abs(gpq - pq) <= H.POOL_TOL * (1 + np.abs(pq)))
    assert np.all(np.abs(gpk - pk) <= H.POOL_TOL * (1 + np.abs(pk)))
    gmask = r["sel"].block_mask.cpu().numpy().astype(bool)
    H.accept_topk_rows(gmask, select.scores(pq, pk), w.topk)
    rp, ci = select.mask_to_csr(gmask)
    assert np.array_equal(r["sel"].row_ptr.cpu().numpy(), rp)
    assert np.array_equal(r["sel"].col_idx.cpu().numpy()[:len(ci)], ci)
    ref, rlse = oatt.block_sparse_attention(tf["q"], tf["k"], tf["v"], gmask, w.T, w.Y, w.X,
                                            tile=T448)
    _check_outputs(w, r, ref, rlse)


@pytest.mark.parametrize("name", ["ragged_d128", "smooth"])
def test_tile128_fused_tile_pool(bsta, name):
    """attn_tile_pool with 128-token tiles: the same tiles and, bit for bit,
    the pooled vectors of the unfused selection; the same CSR."""
    import torch
    w = CASES[name]
    inp = H.inputs(w)
    a = _run(bsta, w, inp)
    b = _run(bsta, w, inp, fused=True)
    assert torch.equal(a["qt"].view(torch.int16), b["qt"].view(torch.int16))
    for x, y in zip(a["sel"].pooled(a["g"]), b["sel"].pooled(b["g"])):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    assert torch.equal(a["sel"].row_ptr, b["sel"].row_ptr)


def test_tile128_oracle_csr_and_dense(bsta):
    """The attention on the oracle's own selection; every tile selected
    equals plain softmax attention (dense float64 brute force)."""
    import torch
    w = CASES["all_tiles"]
    inp = H.inputs(w)
    g = _geom(bsta, w)
    tb, tf = _oracle_tiled(w, inp)
    nt = geometry.num_tiles(w.T, w.Y, w.X, T448)
    assert w.topk == nt
    qt, kt, vt = (H.to_dev(tb[n]) for n in ("q", "k", "v"))
    rng = np.random.default_rng(96)
    om = rng.random((w.B, w.H, nt, nt)) < 0.4
    om[..., 0] = True
    rp, ci = select.mask_to_csr(om)
    ot, lse = bsta.attn_block_sparse_fwd(g, qt, kt, vt, torch.from_numpy(rp).cuda(),
                                         torch.from_numpy(ci).cuda(), want_lse=True)
    o = bsta.attn_block_sparse_fwd(g, qt, kt, vt, torch.from_numpy(rp).cuda(),
                                   torch.from_numpy(ci).cuda(), raster=True)
    torch.cuda.synchronize()
    ref, rlse = oatt.block_sparse_attention(tf["q"], tf["k"], tf["v"], om, w.T, w.Y, w.X, tile=T448)
    _check_outputs(w, dict(ot=ot, lse=lse, o=o), ref, rlse)
    r = _run(bsta, w, inp)
    q, k, v = (workloads.bf16_to_f32(inp[n]) for n in ("q", "k", "v"))
    dense, _ = oatt.dense_masked_attention(q, k, v, np.ones((w.B, w.H, nt, nt), dtype=bool),
                                           w.T, w.Y, w.X, tile=T448)
    H.compare_outputs(H.bf16_dev_to_f32(r["o"]), dense, "all tiles vs dense")


@pytest.mark.parametrize("windows", [[[1, 3, 1], [2, 2, 3]], [[2, 4, 2], [1, 1, 1]]])
def test_tile128_windows(bsta, windows):
    """Sliding tile windows in 128-token tile units: mask and CSR bit-exact,
    attention against the oracle."""
    w = workloads.custom("t128_sta", 1, 2, 128, 8, 16, 24, "sta", seed=97)
    inp = H.inputs(w)
    r = _run(bsta, w, inp, windows=windows)
    om = select.sta_mask(w.T, w.Y, w.X, np.array(windows), w.B, T448)
    assert np.array_equal(r["sel"].block_mask.cpu().numpy().astype(bool), om)
    rp, ci = select.mask_to_csr(om)
    assert np.array_equal(r["sel"].row_ptr.cpu().numpy(), rp)
    _, tf = _oracle_tiled(w, inp)
    ref, rlse = oatt.block_sparse_attention(tf["q"], tf["k"], tf["v"], om, w.T, w.Y, w.X, tile=T448)
    _check_outputs(w, r, ref, rlse)


@pytest.mark.timeout(900)
def test_tile128_full_size(bsta):
    """The 40-head 20x48x80 grid cut into 600 tiles of 4x4x8, top-60 (10%):
    tiles bit-exact, every selection row, and the raster output of one query
    tile per head against the oracle."""
    import torch
    base = workloads.WORKLOADS["c3"]
    w = workloads.Workload("c3_t128", base.index, base.B, base.H, base.D, base.T, base.Y, base.X,
                           "topk", 60, base.structure)
    H.log("128-token tiles, full size: inputs")
    inp = H.inputs(w)
    r = _run(bsta, w, inp, fused=True)
    tb, tf = _oracle_tiled(w, inp)
    assert np.array_equal(H.from_dev(r["qt"]), tb["q"])
    pq = select.pool(tf["q"], w.T, w.Y, w.X, T448)
    pk = select.pool(tf["k"], w.T, w.Y, w.X, T448)
    gmask = r["sel"].block_mask.cpu().numpy().astype(bool)
    exact, band = H.accept_topk_rows(gmask, select.scores(pq, pk), w.topk)
    H.log(f"  rows exact {exact}, inside tie band {band}")
    nt = geometry.num_tiles(w.T, w.Y, w.X, T448)
    rng = np.random.default_rng(98)
    rows = [(0, h, int(rng.integers(nt))) for h in range(w.H)]
    ref, _ = oatt.block_sparse_attention(tf["q"], tf["k"], tf["v"], gmask, w.T, w.Y, w.X, rows=rows,
                                         tile=T448)
    got = H.bf16_dev_to_f32(r["o"])
    assert not torch.isnan(r["o"].float()).any()
    order = geometry.tile_order(w.T, w.Y, w.X, T448)
    gs = [got[b, order[i * 128:(i + 1) * 128], h] for b, h, i in rows]
    rs = [ref[b, i * 128:(i + 1) * 128, h] for b, h, i in rows]
    mx, mean = H.compare_outputs(np.concatenate(gs), np.concatenate(rs), "raster rows")
    H.log(f"  raster rows max-abs {mx:.3g}, mean-abs {mean:.3g}")


def _bwd_run(m, w, inp, r, seed=41):
    import torch
    rng = np.random.default_rng(seed)
    do_bits = workloads.bf16_bits(rng.standard_normal((w.B, w.L, w.H, w.D)).astype(np.float32))
    dot = m.attn_tile(r["g"], H.to_dev(do_bits))
    grads = m.attn_block_sparse_bwd(r["g"], r["qt"], r["kt"], r["vt"], r["ot"], dot, r["lse"],
                                    r["sel"].row_ptr, r["sel"].col_idx)
    torch.cuda.synchronize()
    return do_bits, dot, grads


def _check_bwd(w, grads, tf, dtf, mask, heads=None):
    hs = list(range(w.H)) if heads is None else heads
    sub = lambda a: a[:, :, hs]  # noqa: E731
    args = [sub(tf["q"]), sub(tf["k"]), sub(tf["v"]), sub(dtf)]
    ref = oatt.block_sparse_attention_backward(*args, mask[:, hs], w.T, w.Y, w.X, tile=T448)
    bnd = H.backward_error_bounds(*args, mask[:, hs], w.T, w.Y, w.X, tile=T448)
    valid = np.zeros(ref[0].shape[1], dtype=bool)
    valid[geometry.token_slots(w.T, w.Y, w.X, T448)] = True
    for nm, gt, rf, bd in zip(("dq", "dk", "dv"), grads, ref, bnd):
        bits = H.from_dev(gt)[:, :, hs]
        got = workloads.bf16_to_f32(bits).astype(np.float64)
        err = np.abs(got[:, valid] - rf[:, valid])
        ratio = float((err / (bd[:, valid] + 1e-6)).max())
        H.log(f"  {nm}: max err {err.max():.3g}, max err/bound {ratio:.3f}")
        assert np.all(err <= bd[:, valid] + 1e-6), f"{nm}: error above its bound (ratio {ratio:.3f})"
        assert np.all(bits[:, ~valid] == 0), f"{nm}: pad slots must be +0.0"


@pytest.mark.parametrize("name", sorted(CASES))
def test_tile128_backward(bsta, name):
    """Gradients over 128-token tiles (each tile walked as its two 64-slot
    units, an empty second unit included: the ragged grids end in tiles of
    fewer than 64 tokens) against the oracle's backward with the same tile
    shape, under the GPU's selection; a second call is bitwise equal."""
    w = CASES[name]
    inp = H.inputs(w)
    H.log(f"128-token tiles backward {name}")
    r = _run(bsta, w, inp)
    do_bits, dot, grads = _bwd_run(bsta, w, inp, r)
    _, tf = _oracle_tiled(w, inp)
    dtf = workloads.bf16_to_f32(tiling.tile(do_bits, w.T, w.Y, w.X, T448))
    _check_bwd(w, grads, tf, dtf, r["sel"].block_mask.cpu().numpy().astype(bool))
    again = bsta.attn_block_sparse_bwd(r["g"], r["qt"], r["kt"], r["vt"], r["ot"], dot, r["lse"],
                                       r["sel"].row_ptr, r["sel"].col_idx)
    for a, b in zip(grads, again):
        assert np.array_equal(H.from_dev(a), H.from_dev(b)), "backward is deterministic"


@pytest.mark.parametrize("windows", [[[1, 3, 1], [2, 2, 3]]])
def test_tile128_backward_windows(bsta, windows):
    """Gradients over per-head sliding windows of 128-token tiles (rows of
    different lengths per head)."""
    w = workloads.custom("t128_sta", 1, 2, 128, 8, 16, 24, "sta", seed=97)
    inp = H.inputs(w)
    H.log(f"128-token tiles backward, windows {windows}")
    r = _run(bsta, w, inp, windows=windows)
    do_bits, _, grads = _bwd_run(bsta, w, inp, r)
    _, tf = _oracle_tiled(w, inp)
    dtf = workloads.bf16_to_f32(tiling.tile(do_bits, w.T, w.Y, w.X, T448))
    om = select.sta_mask(w.T, w.Y, w.X, np.array(windows), w.B, T448)
    _check_bwd(w, grads, tf, dtf, om)


@pytest.mark.timeout(900)
def test_tile128_backward_full_size(bsta):
    """The 40-head 20x48x80 grid in 600 tiles of 4x4x8, top-60: every
    gradient of one head against the oracle (the heads are independent)."""
    base = workloads.WORKLOADS["c3"]
    w = workloads.Workload("c3_t128", base.index, base.B, base.H, base.D, base.T, base.Y, base.X,
                           "topk", 60, base.structure)
    H.log("128-token tiles backward, full size")
    inp = H.inputs(w)
    r = _run(bsta, w, inp, fused=True)
    do_bits, _, grads = _bwd_run(bsta, w, inp, r)
    heads = [w.H - 1]
    tf = {n: workloads.bf16_to_f32(tiling.tile(inp[n][:, :, heads], w.T, w.Y, w.X, T448))
          for n in ("q", "k", "v")}
    dtf = workloads.bf16_to_f32(tiling.tile(do_bits[:, :, heads], w.T, w.Y, w.X, T448))
    mask = r["sel"].block_mask.cpu().numpy().astype(bool)[:, heads]
    wsub = workloads.custom("c3_t128_heads", w.B, len(heads), w.D, w.T, w.Y, w.X, "topk", w.topk)
    _check_bwd(wsub, tuple(t[:, :, heads] for t in grads), tf, dtf, mask)
