"""attn_block_sparse_bwd_noalloc (static device scratch, no allocation)
against attn_block_sparse_bwd (caller's workspace), through the C ABI.

Both run the same kernels in the same order, so the gradients must agree bit
for bit.  Two calls in a row use the one scratch array, the second on a
smaller problem, so stale contents of the first call would show; the output
buffers start as NaN so an unwritten element would show too.
"""
import numpy as np
import pytest

import workloads
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

CASES = [workloads.custom("noalloc_big", 1, 12, 128, 16, 32, 32, "topk", 32, "lowrank", seed=51),
         workloads.custom("noalloc_small", 2, 3, 64, 5, 6, 7, "topk", 3, seed=52)]


@pytest.fixture(scope="module")
def bsta():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    import block_sparse_tiled_amd as m
    from block_sparse_tiled_amd import _lib
    _lib.load()
    return m


def _forward(m, w):
    import torch
    inp = workloads.make_inputs(w)
    g = m.Geometry(w.B, w.H, w.D, w.T, w.Y, w.X)
    qt, kt, vt = (m.attn_tile(g, H.to_dev(inp[n])) for n in ("q", "k", "v"))
    sel = m.attn_select_blocks(g, qt, kt, m.SELECT_TOPK, w.topk, want_mask=False)
    ot, lse = m.attn_block_sparse_fwd(g, qt, kt, vt, sel.row_ptr, sel.col_idx, want_lse=True)
    rng = np.random.default_rng(w.index)
    do_bits = workloads.bf16_bits(rng.standard_normal((w.B, w.L, w.H, w.D)).astype(np.float32))
    dot = m.attn_tile(g, H.to_dev(do_bits))
    torch.cuda.synchronize()
    return g, (qt, kt, vt, ot, dot, lse, sel.row_ptr, sel.col_idx)


def test_noalloc_backward_equals_workspace_call(bsta):
    import torch
    for w in CASES:
        H.log(f"noalloc backward: {w.name}")
        g, args = _forward(bsta, w)
        want = bsta.attn_block_sparse_bwd(g, *args)
        got = tuple(torch.full_like(args[0], float("nan")) for _ in range(3))
        bsta.attn_block_sparse_bwd_noalloc(g, *args, out=got)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, want):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{w.name}: {name} differs"


def test_noalloc_backward_capacity(bsta):
    """A CSR capacity whose workspace exceeds the 64 MiB scratch is refused on
    the host with BSTA_ERR_CAPACITY, and nothing is written."""
    import torch
    w = CASES[1]
    g, args = _forward(bsta, w)
    big = torch.zeros(17 << 20, dtype=torch.int32, device="cuda")   # 68 MiB of row_idx alone
    outs = tuple(torch.full_like(args[0], float("nan")) for _ in range(3))
    with pytest.raises(bsta.BstaError) as e:
        bsta.attn_block_sparse_bwd_noalloc(g, *args[:7], big, out=outs)
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert all(torch.isnan(t.float()).all() for t in outs)
