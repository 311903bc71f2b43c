"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: tile/untile, window masks and CSR bit-exact; top-k masks and CSR exact
except rows whose oracle boundary gap is below 1e-4 (which may differ only
inside that band); pooled vectors within 1e-5*(1+|x|); attention outputs
within max-abs 2e-2 and mean-abs 2e-3 over valid rows, pad rows exactly 0.
"""
import math

import numpy as np
import pytest

import workloads
from oracle import attention as oatt
from oracle import geometry, select, tiling
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

SMALL = {
    "c1": workloads.WORKLOADS["c1"],
    "ragged_d128": workloads.custom("ragged_d128", 2, 3, 128, 5, 6, 7, "topk", 3, seed=11),
    "ragged_d64": workloads.custom("ragged_d64", 1, 2, 64, 9, 13, 10, "topk", 5, seed=12),
    "smooth_40": workloads.custom("smooth_40", 1, 4, 128, 8, 16, 20, "topk", 10, "smooth", seed=13),
    "lowrank_48": workloads.custom("lowrank_48", 1, 3, 128, 12, 16, 16, "topk", 6, "lowrank", seed=14),
    "one_token": workloads.custom("one_token", 1, 1, 128, 1, 1, 1, "topk", 1, seed=15),
    "dense_all": workloads.custom("dense_all", 1, 2, 128, 6, 7, 9, "topk", 12, seed=16),
}
STA_SMALL = {
    "sta_small": (workloads.custom("sta_small", 2, 3, 128, 8, 12, 20, "sta", seed=21),
                  [[1, 3, 3], [2, 3, 5], [2, 1, 4]]),
    "sta_ragged": (workloads.custom("sta_ragged", 1, 2, 64, 7, 10, 13, "sta", seed=22),
                   [[2, 3, 4], [1, 1, 1]]),
    "sta_full": (workloads.custom("sta_full", 1, 2, 128, 8, 8, 12, "sta", seed=23),
                 [[2, 2, 3], [2, 2, 3]]),
}


@pytest.fixture(scope="module")
def bsta():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    import block_sparse_tiled_amd as m
    from block_sparse_tiled_amd import _lib
    _lib.load()  # fails loudly when libbsta.so is missing
    return m


def _geom(m, w):
    return m.Geometry(w.B, w.H, w.D, w.T, w.Y, w.X)


def _oracle_tiled(w, inp):
    """Oracle tiling of the bf16 bits, then exact widening to float32."""
    tb = {n: tiling.tile(inp[n], w.T, w.Y, w.X) for n in ("q", "k", "v")}
    tf = {n: workloads.bf16_to_f32(tb[n]) for n in tb}
    return tb, tf


def _run_gpu(m, w, inp, windows=None, want_mask=True):
    import torch
    g = _geom(m, w)
    q, k, v = (H.to_dev(inp[n]) for n in ("q", "k", "v"))
    qt, kt, vt = m.attn_tile(g, q), m.attn_tile(g, k), m.attn_tile(g, v)
    mode = m.SELECT_STA if w.mode == "sta" else m.SELECT_TOPK
    sel = m.attn_select_blocks(g, qt, kt, mode, w.topk, windows, want_mask=want_mask)
    ot, lse = m.attn_block_sparse_fwd(g, qt, kt, vt, sel.row_ptr, sel.col_idx, want_lse=True)
    o = m.attn_untile(g, ot)
    torch.cuda.synchronize()
    return dict(g=g, qt=qt, kt=kt, vt=vt, sel=sel, ot=ot, lse=lse, o=o)


# ---------------------------------------------------------------- tiling

@pytest.mark.parametrize("name", sorted(SMALL))
def test_tile_untile_bit_exact(bsta, name):
    w = SMALL[name]
    inp = H.inputs(w)
    H.log(f"tile/untile {name}")
    g = _geom(bsta, w)
    for n in ("q", "v"):
        x = H.to_dev(inp[n])
        xt = bsta.attn_tile(g, x)
        assert np.array_equal(H.from_dev(xt), tiling.tile(inp[n], w.T, w.Y, w.X))
        back = bsta.attn_untile(g, xt)
        assert np.array_equal(H.from_dev(back), inp[n])


def test_tile_overwrites_stale_padding(bsta):
    """A reused tile buffer full of garbage comes back with zero pad slots."""
    import torch
    w = SMALL["ragged_d128"]
    inp = H.inputs(w)
    g = _geom(bsta, w)
    out = torch.full((w.B, g.Lpad, w.H, w.D), 7.0, dtype=torch.bfloat16, device="cuda")
    bsta.attn_tile(g, H.to_dev(inp["k"]), out=out)
    assert np.array_equal(H.from_dev(out), tiling.tile(inp["k"], w.T, w.Y, w.X))


# ---------------------------------------------------------------- pooling + top-k

@pytest.mark.parametrize("name", sorted(SMALL))
def test_pool_and_topk(bsta, name):
    w = SMALL[name]
    inp = H.inputs(w)
    H.log(f"pool/top-k {name}")
    r = _run_gpu(bsta, w, inp)
    _, tf = _oracle_tiled(w, inp)
    pq = select.pool(tf["q"], w.T, w.Y, w.X)
    pk = select.pool(tf["k"], w.T, w.Y, w.X)
    gpq, gpk = (t.cpu().numpy() for t in r["sel"].pooled(r["g"]))
    for a, b in ((gpq, pq), (gpk, pk)):
        assert np.all(np.abs(a - b) <= H.POOL_TOL * (1 + np.abs(b)))
    s = select.scores(pq, pk)
    gmask = r["sel"].block_mask.cpu().numpy()
    exact, band = H.accept_topk_rows(gmask, s, w.topk)
    H.log(f"  rows exact {exact}, inside tie band {band}")
    # CSR is exactly the GPU mask's rows in ascending order.
    rp, ci = select.mask_to_csr(gmask.astype(bool))
    assert np.array_equal(r["sel"].row_ptr.cpu().numpy(), rp)
    assert np.array_equal(r["sel"].col_idx.cpu().numpy()[:len(ci)], ci)


def test_topk_zero_query_tie_break(bsta):
    """Q = 0: every score is 0 and ties keep tiles 0..k-1 in every row."""
    import torch
    w = SMALL["ragged_d64"]
    g = _geom(bsta, w)
    inp = H.inputs(w)
    q = torch.zeros((w.B, w.L, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    qt, kt = bsta.attn_tile(g, q), bsta.attn_tile(g, H.to_dev(inp["k"]))
    sel = bsta.attn_select_blocks(g, qt, kt, bsta.SELECT_TOPK, 4)
    m = sel.block_mask.cpu().numpy()
    assert np.all(m[..., :4] == 1) and np.all(m[..., 4:] == 0)


# Rows of Nt tiles from a 4 x 4 x 4Nt grid (tile j covers x in [4j, 4j+4)):
# one width in each register bucket of the wave-per-row top-k kernel (at most
# 8, 16, 24 and 32 scores per lane) and one past them (the LDS kernel).
WIDE_NT = [300, 700, 1200, 1900, 2100]


def _select_wide(m, w, q_bits, k_bits):
    g = _geom(m, w)
    qt, kt = m.attn_tile(g, H.to_dev(q_bits)), m.attn_tile(g, H.to_dev(k_bits))
    sel = m.attn_select_blocks(g, qt, kt, m.SELECT_TOPK, w.topk)
    return sel.block_mask.cpu().numpy(), sel.row_ptr.cpu().numpy(), sel.col_idx.cpu().numpy()


def _oracle_scores(w, q_bits, k_bits):
    qt = workloads.bf16_to_f32(tiling.tile(q_bits, w.T, w.Y, w.X))
    kt = workloads.bf16_to_f32(tiling.tile(k_bits, w.T, w.Y, w.X))
    return select.scores(select.pool(qt, w.T, w.Y, w.X), select.pool(kt, w.T, w.Y, w.X))


@pytest.mark.parametrize("nt", WIDE_NT)
def test_topk_wide_rows(bsta, nt):
    """Random inputs: every row accepted against the oracle, CSR = GPU mask rows."""
    w = workloads.custom(f"wide_{nt}", 1, 2, 64, 4, 4, 4 * nt, "topk", nt // 10, seed=31)
    inp = H.inputs(w)
    H.log(f"top-k wide rows Nt={nt} k={w.topk}")
    gmask, rp_g, ci_g = _select_wide(bsta, w, inp["q"], inp["k"])
    s = _oracle_scores(w, inp["q"], inp["k"])
    exact, band = H.accept_topk_rows(gmask, s, w.topk)
    H.log(f"  rows exact {exact}, inside tie band {band}")
    rp, ci = select.mask_to_csr(gmask.astype(bool))
    assert np.array_equal(rp_g, rp)
    assert np.array_equal(ci_g[:len(ci)], ci)


@pytest.mark.parametrize("nt", WIDE_NT)
def test_topk_wide_rows_planted_ties(bsta, nt):
    """Every token of key tile j is c_j * u, c_j in 1..5 (bf16-exact, so the
    pooled key is exactly c_j * u): scores of tiles with equal c_j are equal
    bit for bit on both sides, and wherever the row's sign of q.u is clear
    the kept set must be the oracle's exactly (ties to the lower index)."""
    w = workloads.custom(f"wide_ties_{nt}", 1, 1, 64, 4, 4, 4 * nt, "topk", nt // 7 + 1, seed=41)
    H.log(f"top-k planted ties Nt={nt} k={w.topk}")
    rng = np.random.default_rng(41)
    u = rng.integers(-8, 9, size=w.D).astype(np.float32) / 8.0
    c = ((np.arange(nt) * 7) % 5 + 1).astype(np.float32)
    x = np.arange(w.L) % w.X                 # raster token -> x; tile = x // 4
    kf = (c[x // 4][:, None] * u[None, :]).reshape(1, w.L, 1, w.D)
    k_bits = workloads.bf16_bits(kf)
    assert np.array_equal(workloads.bf16_to_f32(k_bits), kf)
    q_bits = workloads.bf16_bits(rng.standard_normal((1, w.L, 1, w.D)).astype(np.float32))
    gmask, rp_g, ci_g = _select_wide(bsta, w, q_bits, k_bits)
    s = _oracle_scores(w, q_bits, k_bits)
    want = select.topk_mask(s, w.topk)
    # Row i's scores are c_j * (Pq_i . u): rank-clear rows have |Pq_i . u|
    # well above the fp32 rounding of a 64-term dot product.
    qt = workloads.bf16_to_f32(tiling.tile(q_bits, w.T, w.Y, w.X))
    dot = select.pool(qt, w.T, w.Y, w.X)[0, 0] @ u.astype(np.float64)
    clear = np.abs(dot) > 1e-3
    assert clear.sum() > 0.9 * nt
    assert np.array_equal(gmask[0, 0][clear], want[0, 0][clear])
    H.accept_topk_rows(gmask, s, w.topk)
    rp, ci = select.mask_to_csr(gmask.astype(bool))
    assert np.array_equal(rp_g, rp)
    assert np.array_equal(ci_g[:len(ci)], ci)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_tile_pool_fused(bsta, name):
    """attn_tile_pool: the tiled tensor bit for bit attn_tile's (stale rows of
    a reused buffer overwritten), the pooled vectors bit for bit those the
    select call computes itself, and a prepooled selection identical to the
    unfused one."""
    import torch
    w = SMALL[name]
    inp = H.inputs(w)
    H.log(f"tile+pool {name}")
    g = _geom(bsta, w)
    q, k = H.to_dev(inp["q"]), H.to_dev(inp["k"])
    qt, kt = bsta.attn_tile(g, q), bsta.attn_tile(g, k)
    ref = bsta.attn_select_blocks(g, qt, kt, bsta.SELECT_TOPK, w.topk)
    sel = bsta.attn_select_alloc(g, bsta.SELECT_TOPK, w.topk, device=q.device)
    pq, pk = sel.pooled(g)
    qt2 = bsta.attn_tile_pool(g, q, pq, out=torch.full_like(qt, 7.0))
    kt2 = bsta.attn_tile_pool(g, k, pk, out=torch.full_like(kt, 7.0))
    sel = bsta.attn_select_blocks(g, None, None, bsta.SELECT_TOPK | bsta.SELECT_PREPOOLED, w.topk,
                                  out=sel)
    torch.cuda.synchronize()
    for a, b in ((qt2, qt), (kt2, kt)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    rpq, rpk = ref.pooled(g)
    for a, b in ((pq, rpq), (pk, rpk)):
        assert torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))
    # attn_pool (the pooling step on its own) gives the same vectors, and
    # they are the oracle's means
    for x_t, want in ((qt, pq), (kt, pk)):
        got = bsta.attn_pool(g, x_t)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), want.contiguous().view(torch.int32))
    _, tf = _oracle_tiled(w, inp)
    opq = select.pool(tf["q"], w.T, w.Y, w.X)
    assert np.all(np.abs(pq.cpu().numpy() - opq) <= H.POOL_TOL * (1 + np.abs(opq)))
    assert torch.equal(sel.row_ptr, ref.row_ptr)
    nnz = int(ref.row_ptr[-1])
    assert torch.equal(sel.col_idx[:nnz], ref.col_idx[:nnz])
    assert torch.equal(sel.block_mask, ref.block_mask)


@pytest.mark.parametrize("name", ["smooth_40", "ragged_d64", "c1"])
def test_block_sparse_attention_fused_route(bsta, name):
    """The one-call path (Q and K pooled while tiled, prepooled selection)
    equals the four separate calls bit for bit, with the key walk in CSR
    order (deterministic mode); the separate calls are held to the oracle by
    the tests above."""
    import torch
    w = SMALL[name]
    inp = H.inputs(w)
    H.log(f"fused route {name}")
    g = _geom(bsta, w)
    prev = bsta.attn_set_deterministic(True)
    try:
        o = bsta.block_sparse_attention(g, *(H.to_dev(inp[n]) for n in ("q", "k", "v")),
                                        mode=bsta.SELECT_TOPK, topk=w.topk)
        r = _run_gpu(bsta, w, inp)
    finally:
        bsta.attn_set_deterministic(prev)
    assert torch.equal(o.view(torch.int16), r["o"].view(torch.int16))


@pytest.mark.parametrize("name", sorted(SMALL) + sorted(STA_SMALL))
def test_fwd_raster_equals_fwd_then_untile(bsta, name):
    """attn_block_sparse_fwd_raster (output written in raster order, pad slots
    skipped) equals attn_block_sparse_fwd followed by attn_untile bit for bit,
    with the key walk in CSR order; every raster row is written (the buffer
    starts as garbage) and the slot-order lse is the same."""
    import torch
    if name in STA_SMALL:
        w, windows = STA_SMALL[name]
    else:
        w, windows = SMALL[name], None
    inp = H.inputs(w)
    H.log(f"raster output {name}")
    g = _geom(bsta, w)
    prev = bsta.attn_set_deterministic(True)
    try:
        r = _run_gpu(bsta, w, inp, windows=windows, want_mask=False)
        o = torch.full((w.B, w.L, w.H, w.D), 7.0, dtype=torch.bfloat16, device="cuda")
        o, lse = bsta.attn_block_sparse_fwd(g, r["qt"], r["kt"], r["vt"], r["sel"].row_ptr,
                                            r["sel"].col_idx, out=o, want_lse=True, raster=True)
        torch.cuda.synchronize()
    finally:
        bsta.attn_set_deterministic(prev)
    assert torch.equal(o.view(torch.int16), r["o"].view(torch.int16))
    assert torch.equal(lse.view(torch.int32), r["lse"].view(torch.int32))


@pytest.mark.parametrize("name", ["ragged_d128", "smooth_40"])
def test_heads_first_layout(bsta, name):
    """A heads-first [B, H, L, D] layout is the geometry (B*H, 1): every call
    runs unchanged on it.  Its selection is the oracle's (tie band), its
    output (default key walk) matches the oracle's attention under
    that selection, and with the CSR-order walk tiles, CSR and output equal
    those of the standard [B, L, H, D] layout head by head, bit for bit."""
    import torch
    w = SMALL[name]
    inp = H.inputs(w)
    H.log(f"heads-first {name}")
    gh = bsta.Geometry(w.B * w.H, 1, w.D, w.T, w.Y, w.X)
    hf = {n: H.to_dev(inp[n]).permute(0, 2, 1, 3).reshape(w.B * w.H, w.L, 1, w.D).contiguous()
          for n in ("q", "k", "v")}

    def run_hf():
        qt, kt, vt = (bsta.attn_tile(gh, hf[n]) for n in ("q", "k", "v"))
        sel = bsta.attn_select_blocks(gh, qt, kt, bsta.SELECT_TOPK, w.topk)
        o = bsta.attn_block_sparse_fwd(gh, qt, kt, vt, sel.row_ptr, sel.col_idx, raster=True)
        torch.cuda.synchronize()
        return qt, sel, o

    # Against the oracle, in the library's default key walk.
    _, sel, o = run_hf()
    _, tf = _oracle_tiled(w, inp)
    s = select.scores(select.pool(tf["q"], w.T, w.Y, w.X), select.pool(tf["k"], w.T, w.Y, w.X))
    nt = geometry.num_tiles(w.T, w.Y, w.X)
    gmask = sel.block_mask.cpu().numpy().astype(bool).reshape(w.B, w.H, nt, nt)
    H.accept_topk_rows(gmask, s, w.topk)
    ref, _ = oatt.block_sparse_attention(tf["q"], tf["k"], tf["v"], gmask, w.T, w.Y, w.X)
    ref_hf = tiling.untile(ref, w.T, w.Y, w.X).transpose(0, 2, 1, 3).reshape(w.B * w.H, w.L, 1, w.D)
    H.compare_outputs(H.bf16_dev_to_f32(o), ref_hf, "heads-first output")

    # Against the standard layout, bit for bit, with the CSR-order walk.
    prev = bsta.attn_set_deterministic(True)
    try:
        r = _run_gpu(bsta, w, inp, want_mask=False)
        qt, sel, o = run_hf()
    finally:
        bsta.attn_set_deterministic(prev)
    # Heads-first row order (b, h, i) is the standard CSR row order.
    assert torch.equal(sel.row_ptr, r["sel"].row_ptr)
    nnz = int(r["sel"].row_ptr[-1])
    assert torch.equal(sel.col_idx[:nnz], r["sel"].col_idx[:nnz])
    std_tiles = r["qt"].permute(0, 2, 1, 3).reshape(w.B * w.H, -1, 1, w.D)
    assert torch.equal(qt.view(torch.int16), std_tiles.contiguous().view(torch.int16))
    std_o = r["o"].permute(0, 2, 1, 3).reshape(w.B * w.H, w.L, 1, w.D)
    assert torch.equal(o.view(torch.int16), std_o.contiguous().view(torch.int16))


def test_concurrent_calls_on_two_streams(bsta):
    """Two attention calls in flight at once on two streams of equal
    (default) priority, on different inputs and selections.  They share the
    library's per-XCD key-walk counters; each output must still match the
    oracle's attention under its own selection."""
    import torch
    cases = [workloads.custom("two_streams_a", 1, 12, 128, 16, 32, 32, "topk", 32, "lowrank", seed=31),
             workloads.custom("two_streams_b", 1, 8, 128, 12, 40, 36, "topk", 40, "smooth", seed=32)]
    prep = []
    for w in cases:
        inp = workloads.make_inputs(w)
        r = _run_gpu(bsta, w, inp)
        prep.append((w, inp, r))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    prev = bsta.attn_set_key_walk(bsta.WALK_ROTATED)  # both calls use the counters
    try:
        for rep in range(3):
            pair = []
            for (w, inp, r), st in zip(prep, streams):
                with torch.cuda.stream(st):
                    o = torch.full((w.B, w.L, w.H, w.D), float("nan"), dtype=torch.bfloat16,
                                   device="cuda")
                    bsta.attn_block_sparse_fwd(r["g"], r["qt"], r["kt"], r["vt"], r["sel"].row_ptr,
                                               r["sel"].col_idx, out=o, raster=True)
                pair.append(o)
            outs.append(pair)
        torch.cuda.synchronize()
    finally:
        bsta.attn_set_key_walk(prev)
    for n, (w, inp, r) in enumerate(prep):
        H.log(f"two streams: {w.name}")
        _, tf = _oracle_tiled(w, inp)
        gmask = r["sel"].block_mask.cpu().numpy().astype(bool)
        nt = geometry.num_tiles(w.T, w.Y, w.X)
        rows = [(0, h, i) for h in range(w.H) for i in (0, nt // 3, nt - 1)]
        ref, _ = oatt.block_sparse_attention(tf["q"], tf["k"], tf["v"], gmask, w.T, w.Y, w.X,
                                             rows=rows)
        for pair in outs:
            o = pair[n]
            assert not torch.isnan(o.float()).any(), "every raster row is written"
            _compare_raster_rows(w, H.bf16_dev_to_f32(o), ref, rows)


# ---------------------------------------------------------------- windows

@pytest.mark.parametrize("name", sorted(STA_SMALL))
def test_sta_bit_exact(bsta, name):
    w, win = STA_SMALL[name]
    H.log(f"STA {name}")
    g = _geom(bsta, w)
    sel = bsta.attn_select_blocks(g, None, None, bsta.SELECT_STA, 0, win)
    om = select.sta_mask(w.T, w.Y, w.X, np.array(win), w.B)
    assert np.array_equal(sel.block_mask.cpu().numpy().astype(bool), om)
    rp, ci = select.mask_to_csr(om)
    assert np.array_equal(sel.row_ptr.cpu().numpy(), rp)
    assert np.array_equal(sel.col_idx.cpu().numpy(), ci)


@pytest.mark.parametrize("name", sorted(STA_SMALL))
def test_sta_end_to_end(bsta, name):
    w, win = STA_SMALL[name]
    inp = H.inputs(w)
    r = _run_gpu(bsta, w, inp, windows=win)
    _, tf = _oracle_tiled(w, inp)
    om = select.sta_mask(w.T, w.Y, w.X, np.array(win), w.B)
    ref, rlse = oatt.block_sparse_attention(tf["q"], tf["k"], tf["v"], om, w.T, w.Y, w.X)
    H.compare_outputs(H.bf16_dev_to_f32(r["o"]), tiling.untile(ref, w.T, w.Y, w.X))
    _check_tiled_output(w, r, ref, rlse)


# ---------------------------------------------------------------- cumulative threshold

CUM_CASES = [("c1", 0.5, 0), ("ragged_d128", 0.3, 0), ("ragged_d128", 0.9, 2),
             ("ragged_d64", 0.6, 0), ("smooth_40", 0.2, 0), ("smooth_40", 0.95, 5),
             ("lowrank_48", 0.5, 3), ("one_token", 0.5, 0), ("dense_all", 1.0, 0)]


def _check_cumulative(w, sel, s, tau, mb):
    gmask = sel.block_mask.cpu().numpy()
    same, band = H.accept_cumulative_rows(gmask, s, w.D, tau, mb)
    H.log(f"  rows with the oracle's count {same}, inside the mass band {band}")
    rp, ci = select.mask_to_csr(gmask.astype(bool))
    assert np.array_equal(sel.row_ptr.cpu().numpy(), rp)
    assert np.array_equal(sel.col_idx.cpu().numpy()[:len(ci)], ci)
    return gmask.astype(bool)


@pytest.mark.parametrize("name,tau,mb", CUM_CASES)
def test_cumulative_select(bsta, name, tau, mb):
    w = SMALL[name]
    inp = H.inputs(w)
    H.log(f"cumulative {name} threshold {tau} min {mb}")
    g = _geom(bsta, w)
    qt, kt = bsta.attn_tile(g, H.to_dev(inp["q"])), bsta.attn_tile(g, H.to_dev(inp["k"]))
    sel = bsta.attn_select_cumulative(g, qt, kt, tau, mb)
    _check_cumulative(w, sel, _oracle_scores(w, inp["q"], inp["k"]), tau, mb)


@pytest.mark.timeout(900)
def test_cumulative_full_size_c3(bsta):
    """The 40-head 1200-tile workload at the benchmark's threshold (0.15) and
    route (Q and K pooled while tiled): every row of two heads against the
    oracle, and the CSR equal to the GPU mask's rows."""
    import torch
    w = workloads.WORKLOADS["c3"]
    inp = H.inputs(w)
    H.log("cumulative c3 full size")
    g = _geom(bsta, w)
    sel = bsta.attn_select_alloc(g, bsta.SELECT_CUMULATIVE, device="cuda")
    pq, pk = sel.pooled(g)
    bsta.attn_tile_pool(g, H.to_dev(inp["q"]), pq)
    bsta.attn_tile_pool(g, H.to_dev(inp["k"]), pk)
    sel = bsta.attn_select_cumulative(g, None, None, 0.15, 0, prepooled=True, out=sel)
    torch.cuda.synchronize()
    gmask = sel.block_mask.cpu().numpy().astype(bool)
    rp, ci = select.mask_to_csr(gmask)
    assert np.array_equal(sel.row_ptr.cpu().numpy(), rp)
    assert np.array_equal(sel.col_idx[:len(ci)].cpu().numpy(), ci)
    for h in (0, w.H - 1):
        qt = workloads.bf16_to_f32(tiling.tile(inp["q"][:, :, h:h + 1], w.T, w.Y, w.X))
        kt = workloads.bf16_to_f32(tiling.tile(inp["k"][:, :, h:h + 1], w.T, w.Y, w.X))
        s = select.scores(select.pool(qt, w.T, w.Y, w.X), select.pool(kt, w.T, w.Y, w.X))
        same, band = H.accept_cumulative_rows(gmask[:, h:h + 1], s, w.D, 0.15, 0)
        H.log(f"  head {h}: rows with the oracle's count {same}, inside the mass band {band}")


@pytest.mark.parametrize("nt", WIDE_NT[:4])
def test_cumulative_wide_rows(bsta, nt):
    """Random inputs in each register bucket of the one-wave row kernels."""
    w = workloads.custom(f"cwide_{nt}", 1, 2, 64, 4, 4, 4 * nt, "topk", 1, seed=41)
    inp = H.inputs(w)
    s = _oracle_scores(w, inp["q"], inp["k"])
    g = _geom(bsta, w)
    qt, kt = bsta.attn_tile(g, H.to_dev(inp["q"])), bsta.attn_tile(g, H.to_dev(inp["k"]))
    for tau, mb in ((0.1, 0), (0.5, 7), (0.99, 0)):
        H.log(f"cumulative wide Nt={nt} threshold {tau} min {mb}")
        sel = bsta.attn_select_cumulative(g, qt, kt, tau, mb)
        _check_cumulative(w, sel, s, tau, mb)


@pytest.mark.parametrize("nt", [300, 1200])
def test_cumulative_all_ties(bsta, nt):
    """Q = 0: every score is 0, p = 1/Nt, and a row keeps tiles 0..c-1 with c
    the first count whose mass c/Nt reaches the threshold."""
    import torch
    w = workloads.custom(f"cties_{nt}", 1, 2, 64, 4, 4, 4 * nt, "topk", 1, seed=42)
    inp = H.inputs(w)
    g = _geom(bsta, w)
    q = torch.zeros((w.B, w.L, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    qt, kt = bsta.attn_tile(g, q), bsta.attn_tile(g, H.to_dev(inp["k"]))
    for tau in (0.25, 0.5, 0.7):
        sel = bsta.attn_select_cumulative(g, qt, kt, tau, 0)
        m = sel.block_mask.cpu().numpy().reshape(-1, nt).astype(bool)
        c = int(np.ceil(tau * nt - 1e-9))
        cnt = m.sum(axis=1)
        assert np.all(np.abs(cnt - c) <= 1), (tau, np.unique(cnt))
        for r in range(len(m)):
            assert np.all(m[r, :cnt[r]]) and not np.any(m[r, cnt[r]:])


def test_cumulative_small_threshold_equals_topk(bsta):
    """A threshold below every probability keeps max(1, min_blocks) tiles: the
    same CSR, bit for bit, as top-k with that k (one selection kernel)."""
    w = SMALL["smooth_40"]
    inp = H.inputs(w)
    g = _geom(bsta, w)
    qt, kt = bsta.attn_tile(g, H.to_dev(inp["q"])), bsta.attn_tile(g, H.to_dev(inp["k"]))
    for mb in (0, 1, 6):
        c = bsta.attn_select_cumulative(g, qt, kt, 1e-30, mb)
        t = bsta.attn_select_blocks(g, qt, kt, bsta.SELECT_TOPK, max(1, mb))
        n = int(t.row_ptr[-1].item())
        assert np.array_equal(c.row_ptr.cpu().numpy(), t.row_ptr.cpu().numpy())
        assert np.array_equal(c.col_idx[:n].cpu().numpy(), t.col_idx[:n].cpu().numpy())
        assert np.array_equal(c.block_mask.cpu().numpy(), t.block_mask.cpu().numpy())


def test_cumulative_prepooled_equals_pooling(bsta):
    import torch
    w = SMALL["ragged_d128"]
    inp = H.inputs(w)
    g = _geom(bsta, w)
    q, k = H.to_dev(inp["q"]), H.to_dev(inp["k"])
    qt, kt = bsta.attn_tile(g, q), bsta.attn_tile(g, k)
    a = bsta.attn_select_cumulative(g, qt, kt, 0.6, 1)
    sel = bsta.attn_select_alloc(g, bsta.SELECT_CUMULATIVE, device="cuda")
    pq, pk = sel.pooled(g)
    bsta.attn_tile_pool(g, q, pq)
    bsta.attn_tile_pool(g, k, pk)
    b = bsta.attn_select_cumulative(g, None, None, 0.6, 1, prepooled=True, out=sel)
    torch.cuda.synchronize()
    n = int(a.row_ptr[-1].item())
    assert np.array_equal(a.row_ptr.cpu().numpy(), b.row_ptr.cpu().numpy())
    assert np.array_equal(a.col_idx[:n].cpu().numpy(), b.col_idx[:n].cpu().numpy())


def test_cumulative_fused_route(bsta):
    """block_sparse_attention with SELECT_CUMULATIVE (Q and K pooled while
    tiled, prepooled selection) equals the separate calls bit for bit in
    deterministic mode."""
    import torch
    w = SMALL["smooth_40"]
    inp = H.inputs(w)
    g = _geom(bsta, w)
    q, k, v = (H.to_dev(inp[n]) for n in ("q", "k", "v"))
    prev = bsta.attn_set_deterministic(True)
    try:
        o = bsta.block_sparse_attention(g, q, k, v, mode=bsta.SELECT_CUMULATIVE, threshold=0.4,
                                        min_blocks=2)
        qt, kt, vt = bsta.attn_tile(g, q), bsta.attn_tile(g, k), bsta.attn_tile(g, v)
        sel = bsta.attn_select_cumulative(g, qt, kt, 0.4, 2)
        o2 = bsta.attn_block_sparse_fwd(g, qt, kt, vt, sel.row_ptr, sel.col_idx, raster=True)
        torch.cuda.synchronize()
    finally:
        bsta.attn_set_deterministic(prev)
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("name,tau,mb", [("smooth_40", 0.5, 2), ("ragged_d64", 0.8, 0)])
def test_cumulative_end_to_end(bsta, name, tau, mb):
    """Variable-length CSR rows from the cumulative selection feed the
    attention; the oracle attends under the GPU's (validated) mask."""
    import torch
    w = SMALL[name]
    inp = H.inputs(w)
    g = _geom(bsta, w)
    q, k, v = (H.to_dev(inp[n]) for n in ("q", "k", "v"))
    qt, kt, vt = bsta.attn_tile(g, q), bsta.attn_tile(g, k), bsta.attn_tile(g, v)
    sel = bsta.attn_select_cumulative(g, qt, kt, tau, mb)
    o = bsta.attn_block_sparse_fwd(g, qt, kt, vt, sel.row_ptr, sel.col_idx, raster=True)
    torch.cuda.synchronize()
    _, tf = _oracle_tiled(w, inp)
    s = select.scores(select.pool(tf["q"], w.T, w.Y, w.X), select.pool(tf["k"], w.T, w.Y, w.X))
    gmask = _check_cumulative(w, sel, s, tau, mb)
    ref, _ = oatt.block_sparse_attention(tf["q"], tf["k"], tf["v"], gmask, w.T, w.Y, w.X)
    H.compare_outputs(H.bf16_dev_to_f32(o), tiling.untile(ref, w.T, w.Y, w.X))


# ---------------------------------------------------------------- backward

def _run_bwd(m, w, inp, seed=99):
    """Forward (tiled output and lse) and backward on the GPU, dO seeded."""
    import torch
    g = _geom(m, w)
    q, k, v = (H.to_dev(inp[n]) for n in ("q", "k", "v"))
    qt, kt, vt = m.attn_tile(g, q), m.attn_tile(g, k), m.attn_tile(g, v)
    mode = m.SELECT_STA if w.mode == "sta" else m.SELECT_TOPK
    sel = m.attn_select_blocks(g, qt, kt, mode, w.topk, inp.get("windows_list"))
    ot, lse = m.attn_block_sparse_fwd(g, qt, kt, vt, sel.row_ptr, sel.col_idx, want_lse=True)
    rng = np.random.default_rng(seed)
    do_bits = workloads.bf16_bits(rng.standard_normal((w.B, w.L, w.H, w.D)).astype(np.float32))
    dot = m.attn_tile(g, H.to_dev(do_bits))
    grads = m.attn_block_sparse_bwd(g, qt, kt, vt, ot, dot, lse, sel.row_ptr, sel.col_idx)
    torch.cuda.synchronize()
    return dict(g=g, qt=qt, kt=kt, vt=vt, ot=ot, lse=lse, dot=dot, sel=sel, grads=grads,
                do_bits=do_bits)


def _check_grads(w, grads, tf, dtf, mask, heads=None):
    """GPU gradients against the oracle under the per-element bound; pad
    slots exactly zero.  `heads` restricts the check to some heads."""
    hs = list(range(w.H)) if heads is None else heads
    sub = lambda a: a[:, :, hs]  # noqa: E731
    args = [sub(tf["q"]), sub(tf["k"]), sub(tf["v"]), sub(dtf)]
    ref = oatt.block_sparse_attention_backward(*args, mask[:, hs], w.T, w.Y, w.X)
    H.log("  oracle gradients done")
    bnd = H.backward_error_bounds(*args, mask[:, hs], w.T, w.Y, w.X)
    H.log("  error bounds done")
    valid = np.zeros(ref[0].shape[1], dtype=bool)
    valid[geometry.token_slots(w.T, w.Y, w.X)] = True
    for nm, gt, rf, bd in zip(("dq", "dk", "dv"), grads, ref, bnd):
        bits = H.from_dev(gt)[:, :, hs]
        got = workloads.bf16_to_f32(bits).astype(np.float64)
        err = np.abs(got[:, valid] - rf[:, valid])
        ratio = float((err / (bd[:, valid] + 1e-6)).max())
        H.log(f"  {nm}: max err {err.max():.3g}, max err/bound {ratio:.3f}")
        assert np.all(err <= bd[:, valid] + 1e-6), f"{nm}: error above its bound (ratio {ratio:.3f})"
        assert np.all(bits[:, ~valid] == 0), f"{nm}: pad slots must be +0.0"


@pytest.mark.parametrize("name", sorted(SMALL))
def test_backward(bsta, name):
    w = SMALL[name]
    inp = H.inputs(w)
    H.log(f"backward {name}")
    r = _run_bwd(bsta, w, inp)
    _, tf = _oracle_tiled(w, inp)
    dtf = workloads.bf16_to_f32(tiling.tile(r["do_bits"], w.T, w.Y, w.X))
    _check_grads(w, r["grads"], tf, dtf, r["sel"].block_mask.cpu().numpy().astype(bool))


@pytest.mark.parametrize("name", sorted(STA_SMALL))
def test_backward_sta(bsta, name):
    w, win = STA_SMALL[name]
    inp = dict(H.inputs(w), windows_list=win)
    H.log(f"backward {name}")
    r = _run_bwd(bsta, w, inp)
    _, tf = _oracle_tiled(w, inp)
    dtf = workloads.bf16_to_f32(tiling.tile(r["do_bits"], w.T, w.Y, w.X))
    _check_grads(w, r["grads"], tf, dtf, select.sta_mask(w.T, w.Y, w.X, np.array(win), w.B))


def test_backward_on_cumulative_rows(bsta):
    """Gradients over the variable-length rows of the cumulative selection."""
    import torch
    w = SMALL["smooth_40"]
    inp = H.inputs(w)
    g = _geom(bsta, w)
    q, k, v = (H.to_dev(inp[n]) for n in ("q", "k", "v"))
    qt, kt, vt = bsta.attn_tile(g, q), bsta.attn_tile(g, k), bsta.attn_tile(g, v)
    sel = bsta.attn_select_cumulative(g, qt, kt, 0.5, 2)
    ot, lse = bsta.attn_block_sparse_fwd(g, qt, kt, vt, sel.row_ptr, sel.col_idx, want_lse=True)
    rng = np.random.default_rng(17)
    do_bits = workloads.bf16_bits(rng.standard_normal((w.B, w.L, w.H, w.D)).astype(np.float32))
    dot = bsta.attn_tile(g, H.to_dev(do_bits))
    grads = bsta.attn_block_sparse_bwd(g, qt, kt, vt, ot, dot, lse, sel.row_ptr, sel.col_idx)
    torch.cuda.synchronize()
    mask = sel.block_mask.cpu().numpy().astype(bool)
    counts = mask.sum(-1)
    assert counts.min() < counts.max(), "rows should differ in length"
    _, tf = _oracle_tiled(w, inp)
    dtf = workloads.bf16_to_f32(tiling.tile(do_bits, w.T, w.Y, w.X))
    _check_grads(w, grads, tf, dtf, mask)


@pytest.mark.parametrize("mode", ["topk", "cumulative"])
def test_trainable_op_equals_direct_calls(bsta, mode):
    """torch autograd through block_sparse_attention_trainable gives the
    direct calls' output and gradients bit for bit (deterministic mode);
    the direct calls are held to the oracle by the tests above."""
    import torch
    w = SMALL["ragged_d128"]
    inp = H.inputs(w)
    g = _geom(bsta, w)
    q, k, v = (H.to_dev(inp[n]).requires_grad_(True) for n in ("q", "k", "v"))
    m = bsta.SELECT_TOPK if mode == "topk" else bsta.SELECT_CUMULATIVE
    rng = np.random.default_rng(23)
    do_bits = workloads.bf16_bits(rng.standard_normal((w.B, w.L, w.H, w.D)).astype(np.float32))
    do = H.to_dev(do_bits)
    prev = bsta.attn_set_deterministic(True)
    try:
        o = bsta.block_sparse_attention_trainable(g, q, k, v, mode=m, topk=w.topk, threshold=0.5,
                                                  min_blocks=1)
        o.backward(do)
        qt, kt, vt = (bsta.attn_tile(g, t.detach()) for t in (q, k, v))
        sel = (bsta.attn_select_blocks(g, qt, kt, bsta.SELECT_TOPK, w.topk) if mode == "topk"
               else bsta.attn_select_cumulative(g, qt, kt, 0.5, 1))
        ot, lse = bsta.attn_block_sparse_fwd(g, qt, kt, vt, sel.row_ptr, sel.col_idx, want_lse=True)
        grads = bsta.attn_block_sparse_bwd(g, qt, kt, vt, ot, bsta.attn_tile(g, do), lse,
                                           sel.row_ptr, sel.col_idx)
        torch.cuda.synchronize()
    finally:
        bsta.attn_set_deterministic(prev)
    same = lambda a, b: torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))  # noqa: E731
    assert same(o.detach(), bsta.attn_untile(g, ot))
    for t, gr in zip((q, k, v), grads):
        assert same(t.grad, bsta.attn_untile(g, gr))


def test_backward_repeated_ids(bsta):
    """A CSR row that lists a tile twice counts it twice, in the forward and
    in all three gradients: against the chain rule over the row's explicit
    key list, repeats included (the oracle's per-query-tile attention and
    its backward, float64, dK and dV summed per tile)."""
    import torch
    w = SMALL["ragged_d64"]
    inp = H.inputs(w)
    g = _geom(bsta, w)
    _, tf = _oracle_tiled(w, inp)
    nt = geometry.num_tiles(w.T, w.Y, w.X)
    occ = geometry.occupancy(w.T, w.Y, w.X)
    rng = np.random.default_rng(41)
    lists = []
    for r in range(w.B * w.H * nt):
        ids = sorted(rng.choice(nt, size=4, replace=False).tolist())
        if r % 3 == 0:
            ids.insert(1, ids[0])            # a repeat, next to its first occurrence
        if r % 5 == 0:
            ids.append(ids[-1])
        lists.append(ids)
    rp = np.zeros(len(lists) + 1, dtype=np.int32)
    rp[1:] = np.cumsum([len(x) for x in lists])
    ci = np.concatenate(lists).astype(np.int32)
    qt, kt, vt = (H.to_dev(tiling.tile(inp[n], w.T, w.Y, w.X)) for n in ("q", "k", "v"))
    do_bits = workloads.bf16_bits(rng.standard_normal((w.B, w.L, w.H, w.D)).astype(np.float32))
    dot = bsta.attn_tile(g, H.to_dev(do_bits))
    rpd, cid = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    ot, lse = bsta.attn_block_sparse_fwd(g, qt, kt, vt, rpd, cid, want_lse=True)
    grads = bsta.attn_block_sparse_bwd(g, qt, kt, vt, ot, dot, lse, rpd, cid)
    torch.cuda.synchronize()
    dtf = workloads.bf16_to_f32(tiling.tile(do_bits, w.T, w.Y, w.X)).astype(np.float64)
    ref_o = np.zeros(tf["q"].shape)
    ref = [np.zeros(tf["q"].shape) for _ in range(3)]
    bnd = [np.zeros(tf["q"].shape) for _ in range(3)]
    scale = 1.0 / math.sqrt(w.D)
    for r, ids in enumerate(lists):
        b, h, i = r // (w.H * nt), (r // nt) % w.H, r % nt
        rows = slice(i * 64, i * 64 + occ[i])
        keys = np.concatenate([tf["k"][b, j * 64:j * 64 + occ[j], h] for j in ids]).astype(np.float64)
        vals = np.concatenate([tf["v"][b, j * 64:j * 64 + occ[j], h] for j in ids]).astype(np.float64)
        q = tf["q"][b, rows, h].astype(np.float64)
        ref_o[b, rows, h] = oatt.tile_attention(q, keys, vals, scale)[0]
        gq, gk, gv, bq, bk, bv = H.row_backward_bounds(q, keys, vals, dtf[b, rows, h], scale)
        ref[0][b, rows, h] = gq
        bnd[0][b, rows, h] = bq
        at = 0
        for j in ids:
            cols = slice(j * 64, j * 64 + occ[j])
            ref[1][b, cols, h] += gk[at:at + occ[j]]
            ref[2][b, cols, h] += gv[at:at + occ[j]]
            bnd[1][b, cols, h] += bk[at:at + occ[j]]
            bnd[2][b, cols, h] += bv[at:at + occ[j]]
            at += occ[j]
    H.compare_outputs(H.bf16_dev_to_f32(ot), ref_o, "forward with repeated ids")
    for name, gr, rf, bd in zip(("dq", "dk", "dv"), grads, ref, bnd):
        err = np.abs(H.bf16_dev_to_f32(gr).astype(np.float64) - rf)
        bound = bd + H.BF16_U * np.abs(rf) + 1e-6
        assert np.all(err <= bound), f"{name}: error above its bound (ratio {float((err / bound).max()):.3f})"


def test_backward_deterministic(bsta):
    """Fixed summation orders: two calls give bitwise equal gradients."""
    import torch
    w = SMALL["smooth_40"]
    r = _run_bwd(bsta, w, H.inputs(w))
    again = bsta.attn_block_sparse_bwd(r["g"], r["qt"], r["kt"], r["vt"], r["ot"], r["dot"], r["lse"],
                                       r["sel"].row_ptr, r["sel"].col_idx)
    torch.cuda.synchronize()
    for a, b in zip(r["grads"], again):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_backward_unselected_tiles_and_bad_ids(bsta):
    """Key tiles no row selects get zero dK and dV; empty rows get zero dQ;
    out-of-range ids are skipped as in the forward."""
    import torch
    w = SMALL["ragged_d64"]
    inp = H.inputs(w)
    g = _geom(bsta, w)
    nt, lpad = bsta.attn_geometry(g)
    rows = w.B * w.H * nt
    rng = np.random.default_rng(8)
    lists = []
    for r_ in range(rows):
        if r_ % 5 == 0:
            lists.append([])                                   # empty row
        else:
            ids = sorted(rng.choice(nt - 2, size=3, replace=False).tolist())  # tiles nt-2, nt-1 never used
            if r_ % 7 == 0:
                ids = ids + [nt + 5, -1]                       # out of range: skipped
            lists.append(ids)
    rp = np.zeros(rows + 1, dtype=np.int32)
    rp[1:] = np.cumsum([len(x) for x in lists])
    ci = np.array([j for x in lists for j in x], dtype=np.int32)
    q, k, v = (H.to_dev(inp[n]) for n in ("q", "k", "v"))
    qt, kt, vt = bsta.attn_tile(g, q), bsta.attn_tile(g, k), bsta.attn_tile(g, v)
    rpd, cid = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    ot, lse = bsta.attn_block_sparse_fwd(g, qt, kt, vt, rpd, cid, want_lse=True)
    do_bits = workloads.bf16_bits(rng.standard_normal((w.B, w.L, w.H, w.D)).astype(np.float32))
    dot = bsta.attn_tile(g, H.to_dev(do_bits))
    grads = bsta.attn_block_sparse_bwd(g, qt, kt, vt, ot, dot, lse, rpd, cid)
    torch.cuda.synchronize()
    mask = np.zeros((w.B, w.H, nt, nt), dtype=bool)
    for r_, ids in enumerate(lists):
        b, rest = divmod(r_, w.H * nt)
        h, i = divmod(rest, nt)
        for j in ids:
            if 0 <= j < nt:
                mask[b, h, i, j] = True
    _, tf = _oracle_tiled(w, inp)
    dtf = workloads.bf16_to_f32(tiling.tile(do_bits, w.T, w.Y, w.X))
    _check_grads(w, grads, tf, dtf, mask)
    dk = H.from_dev(grads[1])
    assert np.all(dk[:, (nt - 2) * 64:] == 0)


@pytest.mark.timeout(900)
def test_backward_full_size_c3_heads(bsta):
    """The 40-head 1200-tile top-120 workload at full size; every gradient
    of one head against the oracle (the heads are independent)."""
    w = workloads.WORKLOADS["c3"]
    inp = H.inputs(w)
    H.log("backward c3 full size")
    r = _run_bwd(bsta, w, inp)
    heads = [w.H - 1]
    tf = {n: workloads.bf16_to_f32(tiling.tile(inp[n][:, :, heads], w.T, w.Y, w.X))
          for n in ("q", "k", "v")}
    dtf = workloads.bf16_to_f32(tiling.tile(r["do_bits"][:, :, heads], w.T, w.Y, w.X))
    mask = r["sel"].block_mask.cpu().numpy().astype(bool)[:, heads]
    grads = tuple(t[:, :, heads] for t in r["grads"])
    wsub = workloads.custom("c3_heads", w.B, len(heads), w.D, w.T, w.Y, w.X, "topk", w.topk)
    _check_grads(wsub, grads, tf, dtf, mask)


# ---------------------------------------------------------------- attention

def _check_tiled_output(w, r, ref_tiled, ref_lse):
    valid = np.zeros(ref_tiled.shape[1], dtype=bool)
    valid[geometry.token_slots(w.T, w.Y, w.X)] = True
    got = H.bf16_dev_to_f32(r["ot"])
    H.compare_outputs(got[:, valid], ref_tiled[:, valid], "tiled output")
    assert np.all(H.from_dev(r["ot"])[:, ~valid] == 0), "pad rows must be +0.0"
    lse = r["lse"].cpu().numpy()
    assert np.all(np.isneginf(lse[:, :, ~valid]))
    err = np.abs(lse[:, :, valid] - ref_lse[:, :, valid])
    assert err.max() <= H.LSE_TOL, f"lse max err {err.max()}"


@pytest.mark.parametrize("name", sorted(SMALL))
def test_attention_on_oracle_csr(bsta, name):
    """The attention kernel fed with the oracle's own block selection."""
    import torch
    w = SMALL[name]
    inp = H.inputs(w)
    H.log(f"attention on oracle CSR {name}")
    tb, tf = _oracle_tiled(w, inp)
    pq = select.pool(tf["q"], w.T, w.Y, w.X)
    pk = select.pool(tf["k"], w.T, w.Y, w.X)
    om = select.topk_mask(select.scores(pq, pk), w.topk)
    rp, ci = select.mask_to_csr(om)
    g = _geom(bsta, w)
    qt, kt, vt = (H.to_dev(tb[n]) for n in ("q", "k", "v"))
    ot, lse = bsta.attn_block_sparse_fwd(g, qt, kt, vt, torch.from_numpy(rp).cuda(),
                                         torch.from_numpy(ci).cuda(), want_lse=True)
    torch.cuda.synchronize()
    ref, rlse = oatt.block_sparse_attention(tf["q"], tf["k"], tf["v"], om, w.T, w.Y, w.X)
    _check_tiled_output(w, dict(ot=ot, lse=lse), ref, rlse)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_end_to_end(bsta, name):
    """Whole path; the oracle attends under the GPU's (validated) mask."""
    w = SMALL[name]
    inp = H.inputs(w)
    H.log(f"end to end {name}")
    r = _run_gpu(bsta, w, inp)
    _, tf = _oracle_tiled(w, inp)
    gmask = r["sel"].block_mask.cpu().numpy().astype(bool)
    s = select.scores(select.pool(tf["q"], w.T, w.Y, w.X), select.pool(tf["k"], w.T, w.Y, w.X))
    H.accept_topk_rows(gmask, s, w.topk)
    ref, rlse = oatt.block_sparse_attention(tf["q"], tf["k"], tf["v"], gmask, w.T, w.Y, w.X)
    H.compare_outputs(H.bf16_dev_to_f32(r["o"]), tiling.untile(ref, w.T, w.Y, w.X))
    _check_tiled_output(w, r, ref, rlse)


def test_all_tiles_equals_dense_softmax(bsta):
    """k = Nt: the path equals plain softmax attention (oracle brute force)."""
    w = SMALL["dense_all"]
    inp = H.inputs(w)
    nt = geometry.num_tiles(w.T, w.Y, w.X)
    assert w.topk == nt
    r = _run_gpu(bsta, w, inp)
    q, k, v = (workloads.bf16_to_f32(inp[n]) for n in ("q", "k", "v"))
    dense, _ = oatt.dense_masked_attention(q, k, v, np.ones((w.B, w.H, nt, nt), dtype=bool),
                                           w.T, w.Y, w.X)
    H.compare_outputs(H.bf16_dev_to_f32(r["o"]), dense)


def test_empty_rows_and_out_of_range_indices(bsta):
    """Empty CSR rows give zeros / -inf; ids outside [0, Nt) are skipped;
    row ranges past col_len are clamped."""
    import torch
    w = SMALL["ragged_d128"]
    inp = H.inputs(w)
    tb, tf = _oracle_tiled(w, inp)
    nt = geometry.num_tiles(w.T, w.Y, w.X)
    rows = w.B * w.H * nt
    rng = np.random.default_rng(0)
    cols, rp, mask = [], [0], np.zeros((w.B, w.H, nt, nt), dtype=bool)
    for r in range(rows):
        b, rem = divmod(r, w.H * nt)
        h, i = divmod(rem, nt)
        if r % 5 == 0:
            sel = []                       # empty row
        else:
            sel = sorted(rng.choice(nt, size=int(rng.integers(1, nt + 1)), replace=False).tolist())
            mask[b, h, i, sel] = True
            if r % 3 == 0:
                sel = sel + [nt + 3, -1]   # invalid ids, skipped by the kernel
        cols += sel
        rp.append(len(cols))
    g = _geom(bsta, w)
    qt, kt, vt = (H.to_dev(tb[n]) for n in ("q", "k", "v"))
    ot, lse = bsta.attn_block_sparse_fwd(
        g, qt, kt, vt, torch.tensor(rp, dtype=torch.int32, device="cuda"),
        torch.tensor(cols, dtype=torch.int32, device="cuda"), want_lse=True)
    torch.cuda.synchronize()
    ref, rlse = oatt.block_sparse_attention(tf["q"], tf["k"], tf["v"], mask, w.T, w.Y, w.X)
    got = H.bf16_dev_to_f32(ot)
    assert np.all(np.abs(got - ref) <= H.MAX_ABS)
    glse = lse.cpu().numpy()
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(glse), fin)
    assert np.abs(glse[fin] - rlse[fin]).max() <= H.LSE_TOL
    # Truncated col_len: rows past it see fewer tiles, never out-of-bounds reads.
    short = len(cols) // 2
    ot2 = bsta.attn_block_sparse_fwd(
        g, qt, kt, vt, torch.tensor(rp, dtype=torch.int32, device="cuda"),
        torch.tensor(cols[:short], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert np.all(np.isfinite(H.bf16_dev_to_f32(ot2)))


def test_unsorted_empty_and_invalid_rows(bsta):
    """Rows that are empty, unsorted or hold ids outside [0, Nt).  Reversed
    rows put the tiny edge tiles first, where one half of the lanes sees no
    valid key at all: the pair must still share one reference max."""
    import torch
    w = SMALL["ragged_d128"]
    inp = H.inputs(w)
    tb, tf = _oracle_tiled(w, inp)
    nt = geometry.num_tiles(w.T, w.Y, w.X)
    rows = w.B * w.H * nt
    rng = np.random.default_rng(1)
    cols, rp, mask = [], [0], np.zeros((w.B, w.H, nt, nt), dtype=bool)
    for r in range(rows):
        b, rem = divmod(r, w.H * nt)
        h, i = divmod(rem, nt)
        if r % 7 == 0:
            sel = []
        else:
            sel = sorted(rng.choice(nt, size=int(rng.integers(1, nt + 1)), replace=False).tolist())
            mask[b, h, i, sel] = True
            if r % 3 == 0:
                sel = sel[::-1]                 # unsorted row
            if r % 4 == 1:
                sel = [-5] + sel + [nt, nt + 9]  # invalid ids (sorted row stays sorted)
        cols += sel
        rp.append(len(cols))
    g = _geom(bsta, w)
    qt, kt, vt = (H.to_dev(tb[n]) for n in ("q", "k", "v"))
    ref, rlse = oatt.block_sparse_attention(tf["q"], tf["k"], tf["v"], mask, w.T, w.Y, w.X)
    ot, lse = bsta.attn_block_sparse_fwd(
        g, qt, kt, vt, torch.tensor(rp, dtype=torch.int32, device="cuda"),
        torch.tensor(cols, dtype=torch.int32, device="cuda"), want_lse=True)
    torch.cuda.synchronize()
    got = H.bf16_dev_to_f32(ot)
    H.compare_outputs(got, ref)
    glse = lse.cpu().numpy()
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(glse), fin)
    assert np.abs(glse[fin] - rlse[fin]).max() <= H.LSE_TOL


def test_deterministic(bsta):
    """Deterministic mode: equal inputs give bitwise equal outputs."""
    w = SMALL["smooth_40"]
    inp = H.inputs(w)
    prev = bsta.attn_set_deterministic(True)
    try:
        a = _run_gpu(bsta, w, inp)
        b = _run_gpu(bsta, w, inp)
    finally:
        bsta.attn_set_deterministic(prev)
    assert np.array_equal(H.from_dev(a["o"]), H.from_dev(b["o"]))
    assert np.array_equal(a["sel"].col_idx.cpu().numpy(), b["sel"].col_idx.cpu().numpy())


@pytest.mark.parametrize("walk", ["rotated", "auto"])
def test_rotated_walk_matches_deterministic(bsta, walk):
    """The rotated key walk (forced on every row, and the default walk that
    rotates where it pays) differs from the CSR-order walk by rounding only:
    the same selection, outputs within the parity bound of each other, over
    several calls (each starts its rows at different keys)."""
    w = SMALL["smooth_40"]
    inp = H.inputs(w)
    prev = bsta.attn_set_key_walk(bsta.WALK_CSR)
    try:
        assert prev == bsta.WALK_AUTO, "the default mode is the automatic walk"
        ref = _run_gpu(bsta, w, inp)
        bsta.attn_set_key_walk(bsta.WALK_ROTATED if walk == "rotated" else bsta.WALK_AUTO)
        want = H.bf16_dev_to_f32(ref["o"])
        for _ in range(3):
            r = _run_gpu(bsta, w, inp)
            assert np.array_equal(r["sel"].col_idx.cpu().numpy(), ref["sel"].col_idx.cpu().numpy())
            H.compare_outputs(H.bf16_dev_to_f32(r["o"]), want, f"{walk} walk vs CSR order")
    finally:
        bsta.attn_set_key_walk(prev)


# ---------------------------------------------------------------- full sizes

def _compare_raster_rows(w, got_raster, ref_tiled, rows):
    """Raster-order GPU output of query tiles `rows` against the oracle's
    tiled output: the tokens of tile i are the i-th run of the tile order."""
    occ = geometry.occupancy(w.T, w.Y, w.X)
    order = geometry.tile_order(w.T, w.Y, w.X)
    start = np.concatenate([[0], np.cumsum(occ)])
    gs, rs = [], []
    for b, h, i in rows:
        toks = order[start[i]:start[i + 1]]
        gs.append(got_raster[b, toks, h])
        rs.append(ref_tiled[b, i * 64:i * 64 + occ[i], h])
    return H.compare_outputs(np.concatenate(gs), np.concatenate(rs), "raster output rows")


def _csr_mask(row_ptr, col_idx, B, Hh, nt):
    """Block mask of a CSR (host arrays)."""
    mask = np.zeros((B * Hh * nt, nt), dtype=bool)
    for r in range(B * Hh * nt):
        mask[r, col_idx[row_ptr[r]:row_ptr[r + 1]]] = True
    return mask.reshape(B, Hh, nt, nt)


def _full_size_check(bsta, w, inp, n_rows):
    """Full workload through the unfused calls (attn_tile x3, attn_select_blocks
    pooling the tiled Q and K itself, the tiled-output attention, attn_untile);
    selection checked for every row, attention on sampled query tiles.
    Returns the oracle's tiled inputs and scores for the next check."""
    win = inp.get("windows")
    H.log(f"full size {w.name}: GPU path (unfused calls)")
    r = _run_gpu(bsta, w, inp, windows=None if win is None else win.tolist())
    g = r["g"]
    nt = geometry.num_tiles(w.T, w.Y, w.X)
    # tile permutation: bit-exact on Q
    assert np.array_equal(H.from_dev(r["qt"]), tiling.tile(inp["q"], w.T, w.Y, w.X))
    H.log(f"full size {w.name}: oracle selection")
    gmask = r["sel"].block_mask.cpu().numpy().astype(bool)
    tb, tf = _oracle_tiled(w, inp)
    s = pq = pk = None
    if w.mode == "sta":
        om = select.sta_mask(w.T, w.Y, w.X, win, w.B)
        assert np.array_equal(gmask, om)
    else:
        pq = select.pool(tf["q"], w.T, w.Y, w.X)
        pk = select.pool(tf["k"], w.T, w.Y, w.X)
        gpq, gpk = (t.cpu().numpy() for t in r["sel"].pooled(g))
        assert np.all(np.abs(gpq - pq) <= H.POOL_TOL * (1 + np.abs(pq)))
        assert np.all(np.abs(gpk - pk) <= H.POOL_TOL * (1 + np.abs(pk)))
        s = select.scores(pq, pk)
        exact, band = H.accept_topk_rows(gmask, s, w.topk)
        H.log(f"  rows exact {exact}, inside tie band {band}")
    rp, ci = select.mask_to_csr(gmask)
    assert np.array_equal(r["sel"].row_ptr.cpu().numpy(), rp)
    assert np.array_equal(r["sel"].col_idx.cpu().numpy()[:len(ci)], ci)
    H.log(f"full size {w.name}: oracle attention on {n_rows} sampled query tiles")
    rows = H.sample_rows(w.B, w.H, nt, n_rows, seed=w.index)
    ref, rlse = oatt.block_sparse_attention(tf["q"], tf["k"], tf["v"], gmask, w.T, w.Y, w.X,
                                            rows=rows)
    got = H.bf16_dev_to_f32(r["ot"])
    occ = geometry.occupancy(w.T, w.Y, w.X)
    glse = r["lse"].cpu().numpy()
    gs, rs = [], []
    for b, h, i in rows:
        sl = slice(i * 64, i * 64 + occ[i])
        gs.append(got[b, sl, h])
        rs.append(ref[b, sl, h])
        assert np.all(H.from_dev(r["ot"][b, i * 64 + occ[i]:(i + 1) * 64, h]) == 0)
        assert np.abs(glse[b, h, sl] - rlse[b, h, sl]).max() <= H.LSE_TOL
    H.compare_outputs(np.concatenate(gs), np.concatenate(rs))
    # untile of the output is the oracle untile of the GPU's tiled output
    assert np.array_equal(H.from_dev(r["o"]), tiling.untile(H.from_dev(r["ot"]), w.T, w.Y, w.X))
    del r
    return tb, tf, s, pq, pk


def _bench_route(m, w, inp):
    """The benchmark's step, call for call: with top-k, attn_tile_pool tiles Q
    and K and writes their pooled vectors into the selection's workspace,
    attn_tile tiles V, and attn_select_blocks starts from the pooled vectors
    (SELECT_PREPOOLED); with windows, attn_tile tiles all three.  The
    attention writes raster order itself (attn_block_sparse_fwd_raster) in
    the library's default key walk (rotated for the top-k workloads, CSR
    order for windows), into a buffer that starts as
    NaN, so a row left unwritten shows.  No block mask is requested."""
    import torch
    g = _geom(m, w)
    nt, lpad = m.attn_geometry(g)
    mode = m.SELECT_STA if w.mode == "sta" else m.SELECT_TOPK
    win = inp["windows"].tolist() if w.mode == "sta" else None
    q, k, v = (H.to_dev(inp[n]) for n in ("q", "k", "v"))
    qt, kt, vt = (torch.empty((w.B, lpad, w.H, w.D), dtype=torch.bfloat16, device="cuda")
                  for _ in range(3))
    o = torch.full((w.B, w.L, w.H, w.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    sel = m.attn_select_alloc(g, mode, w.topk, win, want_mask=False)
    fused = mode == m.SELECT_TOPK
    if fused:
        pq, pk = sel.pooled(g)
        m.attn_tile_pool(g, q, pq, out=qt)
        m.attn_tile_pool(g, k, pk, out=kt)
    else:
        m.attn_tile(g, q, out=qt)
        m.attn_tile(g, k, out=kt)
    m.attn_tile(g, v, out=vt)
    sel_mode = (m.SELECT_TOPK | m.SELECT_PREPOOLED) if fused else mode
    m.attn_select_blocks(g, None if fused else qt, None if fused else kt, sel_mode, w.topk, win,
                         out=sel)
    m.attn_block_sparse_fwd(g, qt, kt, vt, sel.row_ptr, sel.col_idx, out=o, raster=True)
    torch.cuda.synchronize()
    del q, k, v
    return dict(g=g, qt=qt, kt=kt, vt=vt, sel=sel, o=o)


def _bench_route_check(bsta, w, inp, tb, tf, s, pq, pk):
    """The benchmark's route at full size against the oracle: tiles bit-exact,
    pooled vectors to 1e-5(1+|x|), every selection row (tie band for top-k,
    exact for windows) and the CSR, then the raster attention output of one
    query tile of every (b, h) (plus the first and last tiles) element-wise
    against the oracle's attention under the GPU's validated selection."""
    import torch
    assert bsta.attn_set_deterministic(False) is False, "the default mode is the automatic walk"
    H.log(f"full size {w.name}: benchmark route")
    r = _bench_route(bsta, w, inp)
    g = r["g"]
    nt = geometry.num_tiles(w.T, w.Y, w.X)
    for n in ("q", "k", "v"):
        assert np.array_equal(H.from_dev(r[n + "t"]), tb[n]), f"tiled {n}"
    row_ptr = r["sel"].row_ptr.cpu().numpy().astype(np.int64)
    col_idx = r["sel"].col_idx.cpu().numpy()[:row_ptr[-1]]
    gmask = _csr_mask(row_ptr, col_idx, w.B, w.H, nt)
    if w.mode == "sta":
        assert np.array_equal(gmask, select.sta_mask(w.T, w.Y, w.X, inp["windows"], w.B))
    else:
        gpq, gpk = (t.cpu().numpy() for t in r["sel"].pooled(g))
        assert np.all(np.abs(gpq - pq) <= H.POOL_TOL * (1 + np.abs(pq)))
        assert np.all(np.abs(gpk - pk) <= H.POOL_TOL * (1 + np.abs(pk)))
        exact, band = H.accept_topk_rows(gmask, s, w.topk)
        H.log(f"  rows exact {exact}, inside tie band {band}")
    rp, ci = select.mask_to_csr(gmask)
    assert np.array_equal(row_ptr, rp) and np.array_equal(col_idx, ci), "CSR ascending, row_ptr exact"
    assert not torch.isnan(r["o"].float()).any(), "every raster row is written"
    rng = np.random.default_rng(100 + w.index)
    rows = [(b, h, int(rng.integers(nt))) for b in range(w.B) for h in range(w.H)]
    rows += [(0, 0, 0), (w.B - 1, w.H - 1, nt - 1)]
    H.log(f"full size {w.name}: oracle attention on {len(rows)} query tiles (raster output)")
    ref, _ = oatt.block_sparse_attention(tf["q"], tf["k"], tf["v"], gmask, w.T, w.Y, w.X, rows=rows)
    mx, mean = _compare_raster_rows(w, H.bf16_dev_to_f32(r["o"]), ref, rows)
    H.log(f"  raster rows max-abs {mx:.3g}, mean-abs {mean:.3g}")
    return r


def _oracle_csr_full_head(bsta, w, r, tf, s, h0):
    """The benchmarked attention call (raster output, default walk) on the
    oracle's own top-k selection for head h0, every other row empty: all of
    head h0's query tiles against the oracle; the other heads' rows are zero."""
    import torch
    nt = geometry.num_tiles(w.T, w.Y, w.X)
    om = select.topk_mask(s, w.topk)
    one = np.zeros_like(om)
    one[:, h0] = om[:, h0]
    rp, ci = select.mask_to_csr(one)
    o = torch.full((w.B, w.L, w.H, w.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    bsta.attn_block_sparse_fwd(r["g"], r["qt"], r["kt"], r["vt"], torch.from_numpy(rp).cuda(),
                               torch.from_numpy(ci).cuda(), out=o, raster=True)
    torch.cuda.synchronize()
    H.log(f"full size {w.name}: oracle attention, head {h0}, all {nt} query tiles on the oracle's CSR")
    rows = [(b, h0, i) for b in range(w.B) for i in range(nt)]
    ref, _ = oatt.block_sparse_attention(tf["q"], tf["k"], tf["v"], om, w.T, w.Y, w.X, rows=rows)
    got = H.bf16_dev_to_f32(o)
    mx, mean = _compare_raster_rows(w, got, ref, rows)
    H.log(f"  head {h0}: max-abs {mx:.3g}, mean-abs {mean:.3g}")
    others = np.ones(w.H, dtype=bool)
    others[h0] = False
    assert np.all(H.from_dev(o)[:, :, others] == 0), "empty rows are written as +0.0"


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["c2", "c3", "c4", "c5"])
def test_full_size(bsta, name):
    w = workloads.WORKLOADS[name]
    H.log(f"full size {w.name}: generating inputs")
    inp = H.inputs(w)
    tb, tf, s, pq, pk = _full_size_check(bsta, w, inp, 24)
    r = _bench_route_check(bsta, w, inp, tb, tf, s, pq, pk)
    if name == "c3":
        _oracle_csr_full_head(bsta, w, r, tf, s, h0=17)
