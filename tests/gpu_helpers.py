"""Helpers shared by the GPU parity tests: device transfer, input cache, and
the comparison rules (bit-exact maps, tie band for top-k, max/mean-abs for
attention outputs)."""
from __future__ import annotations

import math

import numpy as np

import workloads
from oracle import select

# Output tolerance for bf16 inputs (max-abs over valid rows, mean-abs).
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
# Top-k sets may differ from the oracle's only where the k-th boundary gap
# of the oracle's scores is below this.
TIE_BAND = 1e-4
# Pooled vectors: |gpu - oracle| <= POOL_TOL * (1 + |oracle|).
POOL_TOL = 1e-5
# Log-sum-exp of valid rows.  The kernel's softmax denominator is the sum of
# the same bf16-rounded probabilities it weights V with (8-bit significand:
# relative rounding error at most 2^-8 each), so its log may be off by up to
# ln(1 + 2^-8) = 3.9e-3 from the exact one, plus fp32 accumulation error.
LSE_TOL = 5e-3

_cache = {}


def inputs(w: workloads.Workload):
    key = (w.name, w.index, w.B, w.H, w.D, w.T, w.Y, w.X, w.structure)
    if key not in _cache:
        if len(_cache) > 2:
            _cache.clear()
        _cache[key] = workloads.make_inputs(w)
    return _cache[key]


def to_dev(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def from_dev(t) -> np.ndarray:
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_dev_to_f32(t) -> np.ndarray:
    return workloads.bf16_to_f32(from_dev(t))


def accept_topk_rows(gpu_mask: np.ndarray, oracle_scores: np.ndarray, k: int):
    """Check every row of a GPU top-k mask against the oracle's scores.

    A row is accepted when its set equals the oracle's set, or when the
    oracle's boundary gap S_(k) - S_(k+1) is below TIE_BAND, the row keeps k
    tiles, every extra tile scores above S_(k) - TIE_BAND and every missing
    tile scores below S_(k+1) + TIE_BAND.  Returns (n_exact, n_band) and
    raises AssertionError on the first failing row.
    """
    om = select.topk_mask(oracle_scores, k)
    gm = gpu_mask.astype(bool)
    nt = oracle_scores.shape[-1]
    s2 = oracle_scores.reshape(-1, nt)
    om2, gm2 = om.reshape(-1, nt), gm.reshape(-1, nt)
    diff_rows = np.nonzero(np.any(om2 != gm2, axis=1))[0]
    if len(diff_rows) == 0:
        return len(s2), 0
    up, lo = select.kth_values(s2[diff_rows], k)
    for n, r in enumerate(diff_rows):
        g, o, s = gm2[r], om2[r], s2[r]
        assert g.sum() == k, f"row {r}: {g.sum()} tiles kept, expected {k}"
        assert up[n] - lo[n] < TIE_BAND, f"row {r}: set differs with gap {up[n] - lo[n]}"
        extra = np.nonzero(g & ~o)[0]
        missing = np.nonzero(o & ~g)[0]
        assert np.all(s[extra] > up[n] - TIE_BAND), f"row {r}: extra tiles {extra}"
        assert np.all(s[missing] < lo[n] + TIE_BAND), f"row {r}: missing tiles {missing}"
    return len(s2) - len(diff_rows), len(diff_rows)


# Probability-mass band of the cumulative-threshold selection (fp32 sums on
# the GPU against the oracle's float64 prefix masses).
MASS_BAND = 1e-4


def accept_cumulative_rows(gpu_mask: np.ndarray, oracle_scores: np.ndarray, D: int,
                           threshold: float, min_blocks: int):
    """Check every row of a GPU cumulative-threshold mask against the oracle.

    A row keeping c tiles is accepted when c >= max(1, min(min_blocks, Nt));
    the oracle's float64 mass of its best c tiles reaches threshold -
    MASS_BAND (or c = Nt); the best c - 1 stay below threshold + MASS_BAND
    (or c is the minimum); and the set is the top-c set up to the top-k tie
    band.  Returns (rows whose count equals the oracle's, rows within the
    band) and raises AssertionError on the first failing row.
    """
    nt = oracle_scores.shape[-1]
    s2 = oracle_scores.reshape(-1, nt)
    gm2 = gpu_mask.astype(bool).reshape(-1, nt)
    cnt = gm2.sum(axis=1)
    kmin = max(1, min(min_blocks, nt))
    masses = select.cumulative_masses(s2, D)
    ocnt = select.cumulative_counts(s2, D, threshold, min_blocks)
    for r in np.nonzero(cnt != ocnt)[0]:
        c = int(cnt[r])
        assert c >= kmin, f"row {r}: {c} tiles kept, below the minimum {kmin}"
        assert c == nt or masses[r, c - 1] >= threshold - MASS_BAND, \
            f"row {r}: {c} tiles hold mass {masses[r, c - 1]:.6f} < {threshold}"
        assert c == kmin or masses[r, c - 2] < threshold + MASS_BAND, \
            f"row {r}: {c - 1} tiles already hold {masses[r, c - 2]:.6f} >= {threshold}"
    for c in np.unique(cnt):
        rows = np.nonzero(cnt == c)[0]
        accept_topk_rows(gm2[rows], s2[rows], int(c))
    same = int((cnt == ocnt).sum())
    return same, len(cnt) - same


# bf16 keeps 8 significand bits, so its unit roundoff (round to nearest) is
# 2^-8: |bf16(x) - x| <= 2^-8 |x|.
BF16_U = 2.0 ** -8


def row_backward_bounds(q, keys, vals, do, scale):
    """Gradients of one query tile over an explicit key list (float64), and
    per-element bounds on the GPU's error in them.

    The GPU recomputes P = exp(s - lse) from the forward's lse (error at
    most LSE_TOL) and rounds it to bf16, so P carries a relative error of
    at most e_P = (exp(LSE_TOL) - 1) + u, u = 2^-8 (bf16's unit roundoff).
    delta = rowsum(dO * O) uses the forward's bf16 output, whose error is
    its rounding (u |O|) plus the forward's own error, at most
    2u * sum_k P_k |V_k| (its weights are bf16-rounded probabilities
    normalised by their own sum).  dS = P (dP - delta) is rounded to bf16.
    Summing absolute values of the terms:
      |err dS| <= (e_P + u) |dS| + (1 + e_P) P |err delta|,
      |err dV| <= e_P * sum_q P |dO|,
      |err dQ| <= scale * sum_keys |err dS| |K|, and the same for dK over
                  the queries with |Q|,
    each gradient adding u times its own magnitude for its final rounding
    (added by the caller, once per summed element).  Products of bf16
    operands are exact in fp32 and fp32 accumulation error is far below
    these terms.  Returns (dq, dkeys, dvals, bound_dq, bound_dkeys, bound_dvals)
    without the final-rounding term.
    """
    u = BF16_U
    e_p = math.expm1(LSE_TOL) + u
    s_ = q @ keys.T * scale
    p = np.exp(s_ - s_.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    o = p @ vals
    ds = p * (do @ vals.T - (do * o).sum(axis=1, keepdims=True))
    err_delta = (np.abs(do) * (u * np.abs(o) + 2.0 * u * (p @ np.abs(vals)))).sum(axis=1, keepdims=True)
    eds = (e_p + u) * np.abs(ds) + (1.0 + e_p) * p * err_delta
    return (scale * ds @ keys, scale * ds.T @ q, p.T @ do,
            scale * eds @ np.abs(keys), scale * eds.T @ np.abs(q), e_p * p.T @ np.abs(do))


def backward_error_bounds(qt, kt, vt, dot, mask, T, Y, X, occ=None, tile=None):
    """Per-element error bounds for the GPU gradients (float64, tiled shapes):
    row_backward_bounds summed over the selection, plus the final bf16
    rounding of each gradient (u times its magnitude).  ``occ`` (valid
    tokens per tile) replaces the (T, Y, X) grid's, e.g. for a packed
    sequence; ``tile`` is the tile shape (default 4x4x4).  Returns
    (bound_dq, bound_dk, bound_dv)."""
    from oracle import geometry as ogeo
    u = BF16_U
    B, lpad, Hh, D = qt.shape
    tile = ogeo.TILE if tile is None else tile
    E = ogeo.tile_elems(tile)
    if occ is None:
        occ = ogeo.occupancy(T, Y, X, tile)
    scale = 1.0 / np.sqrt(D)
    bq, bk, bv = (np.zeros((B, lpad, Hh, D)) for _ in range(3))
    gq, gk, gv = (np.zeros((B, lpad, Hh, D)) for _ in range(3))
    for b in range(B):
        for h in range(Hh):
            for i in range(len(occ)):
                sel = np.nonzero(mask[b, h, i])[0]
                if len(sel) == 0:
                    continue
                rows = slice(i * E, i * E + occ[i])
                q = qt[b, rows, h].astype(np.float64)
                do = dot[b, rows, h].astype(np.float64)
                keys = np.concatenate([kt[b, j * E:j * E + occ[j], h] for j in sel]).astype(np.float64)
                vals = np.concatenate([vt[b, j * E:j * E + occ[j], h] for j in sel]).astype(np.float64)
                cgq, cgk, cgv, cbq, cbk, cbv = row_backward_bounds(q, keys, vals, do, scale)
                gq[b, rows, h] = cgq
                bq[b, rows, h] = cbq
                at = 0
                for j in sel:
                    cols = slice(j * E, j * E + occ[j])
                    bk[b, cols, h] += cbk[at:at + occ[j]]
                    bv[b, cols, h] += cbv[at:at + occ[j]]
                    gk[b, cols, h] += cgk[at:at + occ[j]]
                    gv[b, cols, h] += cgv[at:at + occ[j]]
                    at += occ[j]
    return bq + u * np.abs(gq), bk + u * np.abs(gk), bv + u * np.abs(gv)


def compare_outputs(gpu: np.ndarray, ref: np.ndarray, what: str = "output"):
    """Max-abs and mean-abs bounds between two float arrays of valid rows."""
    err = np.abs(gpu.astype(np.float64) - ref.astype(np.float64))
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{what}: max-abs {mx:.3g}, mean-abs {mean:.3g}"
    return mx, mean


def sample_rows(B, H, nt, n, seed=0):
    rng = np.random.default_rng(seed)
    rows = {(0, 0, 0), (B - 1, H - 1, nt - 1)}
    while len(rows) < min(n, B * H * nt):
        rows.add((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(nt))))
    return sorted(rows)


def log(msg):
    print(msg, flush=True)


def scale_of(D):
    return 1.0 / math.sqrt(D)
