"""Benchmark of the block-sparse tiled attention path on one MI355X.

One step = the whole path on one batch already resident in HBM:
tile Q, K, V -> select blocks (pool, score, top-k -> CSR) -> block-sparse
attention forward -> untile O.  Prints one JSON line.

Default workload: B=1, H=40, D=128, latent 20x48x80 (L=76,800, 1200 tiles of
4x4x4), top-k 120 key tiles per query tile, Q/K/V ~ N(0,1) plus a shared
Gaussian-blurred (sigma 2 tokens) component at 0.5 amplitude.

value = selected-tile attention FLOP per step / step time (whole path),
in TFLOP/s.  The attention kernel's own rate is in "roofline" and
"kernels.attn_fwd".  Kernel times come from HIP events recorded on the
stream every call is enqueued on (torch's current stream).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
# Threshold of the cumulative-threshold selection timed beside the step: on
# the synthetic 40-head 1200-tile workload it keeps about 10% of the key
# tiles, the density of its top-120 selection.
CUM_THRESHOLD = 0.15
# Keep ratio of the query-pruning leg timed beside the step.
PRUNE_RATIO = 0.5
METRIC = "block-sparse attn fwd ms/call + TFLOP/s (frac of bf16 MFMA peak), 1 MI355X"

# Counter readings of the attention kernel on the default workload, from the
# rocprofv3 summaries under profiles/ (attn_path_c3_counters.txt, and
# attn_fwd_c3_instruction_mix.txt for the instructions per key tile and wave).  HBM bytes per
# launch = FETCH_SIZE KiB * 1024 * 2.0 + WRITE_SIZE KiB * 1024 * 1.0, the
# factors read off a plain 1 GiB copy (copy_1GiB_hbm_calibration.txt).  The
# readings hold only for the kernel source they were taken on: when
# attn_fwd.hip no longer hashes to "src_sha256_16" they are reported as null.
MEASURED_ATTN = {
    "src_sha256_16": "8d74cb5a45bdd315",
    "fetch_kib": 37409783, "write_kib": 792684, "traffic_bytes": 77426943184,
    "l2_hit": 0.604, "lds_bank_conflict_per_active": 0.0,
    "mfma_busy": 0.464, "clock_ghz": 1.674,
    "insts_per_key_tile_wave": {"valu": 194.1, "mfma": 32.0, "salu": 117.9, "lds": 48.0,
                                "branch": 25.3, "vmem": 16.3, "smem": 1.0},
}


def measured_attn():
    """MEASURED_ATTN if the kernel source still matches it, else None."""
    import hashlib
    src = os.path.join(ROOT, "block_sparse_tiled_amd", "csrc", "attn_fwd.hip")
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    return MEASURED_ATTN if sha == MEASURED_ATTN["src_sha256_16"] else None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="c3", choices=["c1", "c2", "c3", "c4", "c5"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--deterministic", action="store_true",
                   help="walk every CSR row in order (attn_set_deterministic) instead of the "
                        "default rotated key walk")
    p.add_argument("--legs", default="all", choices=["all", "step", "bwd"],
                   help="step: time only the step and its per-call events (for profiling the "
                        "step's kernels without the side measurements' other workloads); bwd: "
                        "the step and the backward leg")
    p.add_argument("--mode", default="path", choices=["path", "copy"],
                   help="copy: time a plain 1 GiB device copy (HBM counter calibration)")
    return p.parse_args()


def copy_calibration(steps: int):
    """A plain device-to-device copy of a known size: the reference for scaling
    the FETCH_SIZE / WRITE_SIZE counters of the path's kernels."""
    import torch
    n = 1 << 29  # bf16 elements = 1 GiB
    x = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    for _ in range(2):
        y.copy_(x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        y.copy_(x)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"mode": "copy", "bytes_read": 2 * n, "bytes_written": 2 * n,
                      "ms": dt * 1e3, "gbps": 4 * n / dt / 1e9}), flush=True)


def attention_flop(w, mask_rows_nnz, occupancy=None):
    """4*D*64*64 per selected (query tile, key tile) pair (tile level)."""
    return 4.0 * w.D * 64 * 64 * mask_rows_nnz


def cpu_baseline(w):
    """The oracle, as it stands, on one head of the workload (all its query tiles)."""
    import numpy as np
    import workloads
    from oracle import geometry, pipeline
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    w1 = workloads.custom(w.name + "_1head", w.B, 1, w.D, w.T, w.Y, w.X, w.mode, w.topk,
                          w.structure, seed=w.seed)
    inp = workloads.make_inputs(w1)
    win = None
    if w.mode == "sta":
        win = workloads.sta_windows(w)[:1]
    t0 = time.perf_counter()
    res = pipeline.run(inp["q"], inp["k"], inp["v"], w.T, w.Y, w.X, w.mode, w.topk, win)
    dt = time.perf_counter() - t0
    flop = attention_flop(w, int(res["mask"].sum()))
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"1 of {w.H} heads, all {geometry.num_tiles(w.T, w.Y, w.X)} query tiles, "
                      f"whole oracle path (tile, pool, score, select, attend, untile), float64 numpy",
            "seconds": dt, "os_cpu_count": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0))}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.mode == "copy":
        copy_calibration(args.steps)
        return
    import numpy as np
    import torch

    import block_sparse_tiled_amd as bsta
    import workloads

    bsta.attn_set_deterministic(args.deterministic)
    w = workloads.WORKLOADS[args.workload]
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    inp = workloads.make_inputs(w)
    g = bsta.Geometry(w.B, w.H, w.D, w.T, w.Y, w.X)
    dev = torch.device("cuda:0")

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    nt, lpad = bsta.attn_geometry(g)
    mode = bsta.SELECT_STA if w.mode == "sta" else bsta.SELECT_TOPK
    win = inp["windows"].tolist() if w.mode == "sta" else None
    # Preallocated outputs: the timed region allocates nothing.
    qt, kt, vt, ot = (torch.empty((w.B, lpad, w.H, w.D), dtype=torch.bfloat16, device=dev)
                      for _ in range(4))
    pool_q, pool_k = (torch.empty((w.B, w.H, nt, w.D), dtype=torch.float32, device=dev)
                      for _ in range(2))
    o = torch.empty_like(q)
    sel = bsta.attn_select_alloc(g, mode, w.topk, win, want_mask=False, device=dev)
    # Top-k: Q and K are pooled in the tiling pass (attn_tile_pool writes the
    # pooled vectors into the selection's workspace) and the selection skips
    # its own pooling pass.
    fused = mode == bsta.SELECT_TOPK
    pq, pk = sel.pooled(g) if fused else (None, None)
    sel_mode = (bsta.SELECT_TOPK | bsta.SELECT_PREPOOLED) if fused else mode
    # The attention call writes its output in raster order itself
    # (attn_block_sparse_fwd_raster), so the step has no untile pass.
    names = ["tile_qk", "tile_v", "select", "attn_fwd"]
    # In the timed steps V is tiled on a second stream (default priority)
    # while the selection runs on the main one: the selection does not read
    # V, and the attention waits for both.  The side stream first waits for
    # the main stream, so V's tiling also follows the previous step's
    # attention, which reads the same tiled buffer.  The per-call timing
    # below runs every call in order on the main stream.
    side = torch.cuda.Stream(device=dev)
    v_done = torch.cuda.Event()

    def step_overlapped():
        main = torch.cuda.current_stream(dev)
        if fused:
            bsta.attn_tile_pool(g, q, pq, out=qt)
            bsta.attn_tile_pool(g, k, pk, out=kt)
        else:
            bsta.attn_tile(g, q, out=qt)
            bsta.attn_tile(g, k, out=kt)
        side.wait_stream(main)
        with torch.cuda.stream(side):
            bsta.attn_tile(g, v, out=vt)
            v_done.record(side)
        bsta.attn_select_blocks(g, None if fused else qt, None if fused else kt, sel_mode, w.topk,
                                win, out=sel)
        main.wait_event(v_done)
        bsta.attn_block_sparse_fwd(g, qt, kt, vt, sel.row_ptr, sel.col_idx, out=o, raster=True)

    def step(ev=None):
        if ev:
            ev[0].record()
        if fused:
            bsta.attn_tile_pool(g, q, pq, out=qt)
            bsta.attn_tile_pool(g, k, pk, out=kt)
        else:
            bsta.attn_tile(g, q, out=qt)
            bsta.attn_tile(g, k, out=kt)
        if ev:
            ev[1].record()
        bsta.attn_tile(g, v, out=vt)
        if ev:
            ev[2].record()
        bsta.attn_select_blocks(g, None if fused else qt, None if fused else kt, sel_mode, w.topk,
                                win, out=sel)
        if ev:
            ev[3].record()
        bsta.attn_block_sparse_fwd(g, qt, kt, vt, sel.row_ptr, sel.col_idx, out=o, raster=True)
        if ev:
            ev[4].record()

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step_overlapped()
    torch.cuda.synchronize()
    nnz = int(sel.row_ptr[-1].item())

    # Whole-step timing (no per-kernel events inside).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step_overlapped()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # Per-call timing with HIP events on the launch stream: the median of at
    # least 20 calls of each.
    n_calls = max(args.steps, 20)
    per = {n: [] for n in names}
    for _ in range(n_calls):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        step(ev)
        torch.cuda.synchronize()
        for idx, n in enumerate(names):
            per[n].append(ev[idx].elapsed_time(ev[idx + 1]))
    ms = {n: float(np.median(per[n])) for n in names}
    ms["tile_qkv"] = float(np.median([a + b for a, b in zip(per["tile_qk"], per["tile_v"])]))
    print(f"[bench] per-call median ms {ms}", file=sys.stderr, flush=True)

    # The pooling step on its own (attn_pool on the tiled Q and K), for its
    # HBM rate; not part of the step (the step pools while tiling).
    per_pool = []
    for _ in range(n_calls):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        bsta.attn_pool(g, qt, out=pool_q)
        bsta.attn_pool(g, kt, out=pool_k)
        e1.record()
        torch.cuda.synchronize()
        per_pool.append(e0.elapsed_time(e1))
    pool_ms = float(np.median(per_pool))

    # Valid-token work of the step's selection: 4*D*n_i*n_j per selected
    # pair (n = valid tokens per tile), against the tile-level 4*D*64*64.
    occ_t = torch.tensor(bsta.attn_geometry(g, with_occupancy=True)[2], dtype=torch.float64,
                         device=dev)
    rp64 = sel.row_ptr.to(torch.int64)
    row_len = rp64[1:] - rp64[:-1]
    row_tile = torch.arange(w.B * w.H * nt, device=dev) % nt
    n_i = torch.repeat_interleave(occ_t[row_tile], row_len)
    n_j = occ_t[sel.col_idx[:int(rp64[-1].item())].to(torch.int64)]
    valid_flop = float(4.0 * w.D * (n_i * n_j).sum().item())

    # The unfused selection (its own pooling pass over the tiled Q and K), for
    # the pooling kernel's standalone rate; not part of the step.
    unfused_ms = None
    if fused:
        sel_u = bsta.attn_select_alloc(g, mode, w.topk, want_mask=False, device=dev)
        per_u = []
        for _ in range(n_calls):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            bsta.attn_select_blocks(g, qt, kt, mode, w.topk, out=sel_u)
            e1.record()
            torch.cuda.synchronize()
            per_u.append(e0.elapsed_time(e1))
        unfused_ms = float(np.median(per_u))
        del sel_u

    # The side measurements below run other attention workloads (the tiled
    # output, cold caches, other selections and geometries); --legs step
    # leaves them out.
    legs = args.legs == "all"
    bwd_leg = args.legs in ("all", "bwd")

    # The standalone untile pass (not in the step: the attention writes raster
    # order itself), for its HBM rate.
    untile_ms = cold_ms = None
    if legs:
        bsta.attn_block_sparse_fwd(g, qt, kt, vt, sel.row_ptr, sel.col_idx, out=ot)
        per_ut = []
        for _ in range(n_calls):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            bsta.attn_untile(g, ot, out=o)
            e1.record()
            torch.cuda.synchronize()
            per_ut.append(e0.elapsed_time(e1))
        untile_ms = float(np.median(per_ut))

    # Cold-L2 row for the attention call: a 512 MB write before each call
    # evicts the key/value tiles a previous call left in the caches.
    if legs:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cold = []
        for _ in range(n_calls):
            flush.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            bsta.attn_block_sparse_fwd(g, qt, kt, vt, sel.row_ptr, sel.col_idx, out=o, raster=True)
            e1.record()
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        del flush
        cold_ms = float(np.median(cold))
        print(f"[bench] attention cold-L2 median ms {cold_ms:.3f}", file=sys.stderr, flush=True)

    # The cumulative-threshold selection (attn_select_cumulative) on the same
    # pooled Q and K, and the attention over its variable-length rows; not
    # part of the step.
    cum = None
    if legs and fused and nt <= 2048:
        sel_c = bsta.attn_select_alloc(g, bsta.SELECT_CUMULATIVE, want_mask=False, device=dev)
        cq, ck = sel_c.pooled(g)
        cq.copy_(pq)
        ck.copy_(pk)
        per_c, per_ca = [], []
        for _ in range(n_calls):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            bsta.attn_select_cumulative(g, None, None, CUM_THRESHOLD, 0, prepooled=True, out=sel_c)
            e[1].record()
            bsta.attn_block_sparse_fwd(g, qt, kt, vt, sel_c.row_ptr, sel_c.col_idx, out=o,
                                       raster=True)
            e[2].record()
            torch.cuda.synchronize()
            per_c.append(e[0].elapsed_time(e[1]))
            per_ca.append(e[1].elapsed_time(e[2]))
        nnz_c = int(sel_c.row_ptr[-1].item())
        c_ms, ca_ms = float(np.median(per_c)), float(np.median(per_ca))
        cum = {"ms": c_ms, "threshold": CUM_THRESHOLD, "min_blocks": 0,
               "selected_tile_pairs": nnz_c, "density": nnz_c / float(w.B * w.H * nt * nt),
               "attn_ms": ca_ms,
               "attn_tflops": attention_flop(w, nnz_c) / (ca_ms * 1e-3) / 1e12,
               "note": "scores + cumulative-threshold counts and ids + row scan + compaction (prepooled); "
                       "attention over its rows; not in the step"}
        print(f"[bench] cumulative selection {cum}", file=sys.stderr, flush=True)
        del sel_c

    # Query pruning (attn_prune_queries) at keep ratio 0.5 on the tiled Q,
    # the cumulative-threshold selection from the kept queries' means, and
    # the pruned attention (attn_block_sparse_fwd_pruned); not part of the
    # step.  Pruned rows are masked in the attention, not skipped.
    pruned = None
    if legs and fused and nt <= 2048:
        sel_p = bsta.attn_select_alloc(g, bsta.SELECT_CUMULATIVE, want_mask=False, device=dev)
        ppq, ppk = sel_p.pooled(g)
        ppk.copy_(pk)
        keep = torch.empty((w.B, w.H, nt), dtype=torch.int64, device=dev)
        kcount = torch.empty((w.B, w.H, nt), dtype=torch.int32, device=dev)
        per_p = {"prune": [], "select": [], "attn": []}
        for _ in range(n_calls):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            e[0].record()
            bsta.attn_prune_queries(g, qt, PRUNE_RATIO, pooled=ppq, keep_mask=keep, keep_count=kcount)
            e[1].record()
            bsta.attn_select_cumulative(g, None, None, CUM_THRESHOLD, 0, prepooled=True, out=sel_p)
            e[2].record()
            bsta.attn_block_sparse_fwd(g, qt, kt, vt, sel_p.row_ptr, sel_p.col_idx, out=o,
                                       raster=True, keep=keep)
            e[3].record()
            torch.cuda.synchronize()
            for idx, n in enumerate(per_p):
                per_p[n].append(e[idx].elapsed_time(e[idx + 1]))
        nnz_p = int(sel_p.row_ptr[-1].item())
        pms = {n: float(np.median(v)) for n, v in per_p.items()}
        q_bytes = w.B * w.H * w.D * 2 * lpad + w.B * w.H * nt * (w.D * 4 + 12)
        pruned = {"keep_ratio": PRUNE_RATIO, "threshold": CUM_THRESHOLD,
                  "prune_ms": pms["prune"], "prune_gbps": q_bytes / (pms["prune"] * 1e-3) / 1e9,
                  "select_ms": pms["select"], "attn_ms": pms["attn"],
                  "selected_tile_pairs": nnz_p,
                  "attn_tflops_kept_rows": PRUNE_RATIO * attention_flop(w, nnz_p) / (pms["attn"] * 1e-3) / 1e12,
                  "note": "prune (scores, ranks, kept means) + cumulative selection from the kept means + "
                          "attention writing kept rows (pruned rows masked, not skipped); not in the step"}
        print(f"[bench] pruned queries {pruned}", file=sys.stderr, flush=True)
        del sel_p, keep, kcount

    # 128-token tiles (4x4x8) on the same raster inputs: the step's calls with
    # a geometry of half as many tiles and top-k halved (same density); not
    # part of the step.
    t128 = None
    if legs and w.mode == "topk":
        g8 = bsta.Geometry(w.B, w.H, w.D, w.T, w.Y, w.X, tile_x=8)
        nt8, lpad8 = bsta.attn_geometry(g8)
        k8 = max(1, min(nt8, w.topk * nt8 // nt))
        qt8, kt8, vt8 = (torch.empty((w.B, lpad8, w.H, w.D), dtype=torch.bfloat16, device=dev)
                         for _ in range(3))
        sel8 = bsta.attn_select_alloc(g8, bsta.SELECT_TOPK, k8, want_mask=False, device=dev)
        pq8, pk8 = sel8.pooled(g8)
        per8 = {"tile_qkv": [], "select": [], "attn_fwd": []}
        for it in range(n_calls + 2):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            e[0].record()
            bsta.attn_tile_pool(g8, q, pq8, out=qt8)
            bsta.attn_tile_pool(g8, k, pk8, out=kt8)
            bsta.attn_tile(g8, v, out=vt8)
            e[1].record()
            bsta.attn_select_blocks(g8, None, None, bsta.SELECT_TOPK | bsta.SELECT_PREPOOLED, k8,
                                    out=sel8)
            e[2].record()
            bsta.attn_block_sparse_fwd(g8, qt8, kt8, vt8, sel8.row_ptr, sel8.col_idx, out=o,
                                       raster=True)
            e[3].record()
            torch.cuda.synchronize()
            if it >= 2:
                for idx, n in enumerate(per8):
                    per8[n].append(e[idx].elapsed_time(e[idx + 1]))
        nnz8 = int(sel8.row_ptr[-1].item())
        ms8 = {n: float(np.median(v_)) for n, v_ in per8.items()}
        flop8 = 4.0 * w.D * 128 * 128 * nnz8
        # The backward over the same selection (tiled output and lse from one
        # more forward call, a seeded dO): five products per selected pair.
        b8 = None
        if nt8 <= 4096:
            ot8, lse8 = bsta.attn_block_sparse_fwd(g8, qt8, kt8, vt8, sel8.row_ptr, sel8.col_idx,
                                                   want_lse=True)
            gen8 = torch.Generator(device=dev).manual_seed(7)
            dot8 = torch.randn(ot8.shape, generator=gen8, device=dev).to(torch.bfloat16)
            gr8 = tuple(torch.empty_like(qt8) for _ in range(3))
            per_b8 = []
            for it in range(4):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                bsta.attn_block_sparse_bwd(g8, qt8, kt8, vt8, ot8, dot8, lse8, sel8.row_ptr,
                                           sel8.col_idx, out=gr8)
                e1.record()
                torch.cuda.synchronize()
                if it >= 1:
                    per_b8.append(e0.elapsed_time(e1))
            b8 = float(np.median(per_b8))
            del ot8, lse8, dot8, gr8
        t128 = {"tile": [4, 4, 8], "tiles": nt8, "topk": k8, "selected_tile_pairs": nnz8,
                "tile_qkv_ms": ms8["tile_qkv"], "select_ms": ms8["select"],
                "attn_ms": ms8["attn_fwd"],
                "attn_tflops": flop8 / (ms8["attn_fwd"] * 1e-3) / 1e12,
                "attn_frac_mfma_peak": flop8 / (ms8["attn_fwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                "bwd_ms": b8,
                "bwd_tflops": None if b8 is None else 2.5 * flop8 / (b8 * 1e-3) / 1e12,
                "note": "128-token tiles: tile_pool/tile, top-k from pooled, raster attention "
                        "(each 128-key tile = two 64-key units); the backward walks the same "
                        "units (3 timed calls, median); not in the step"}
        print(f"[bench] 128-token tiles {t128}", file=sys.stderr, flush=True)
        del qt8, kt8, vt8, sel8

    # A packed sequence (reading of the "video_sparse_attn_h3" page's build()):
    # a 226-row dense prefix, a 4xYxX reference region kept at 0.5 and the
    # step's grid as the generated region at sparsity 0.9, on seeded N(0,1)
    # inputs: tile+pool, packed selection (exempt), raster attention; not
    # part of the step.
    packed_leg = None
    if legs and args.workload == "c3":
        segs = [226, (4, w.Y, w.X), (w.T, w.Y, w.X)]
        gp = bsta.Geometry.packed(w.B, w.H, w.D, segs)
        ntp, lpadp = bsta.attn_geometry(gp)
        info = bsta.attn_packed_info(gp)
        gen = torch.Generator(device=dev).manual_seed(11)
        qp, kp, vp = (torch.randn((w.B, info["L"], w.H, w.D), generator=gen, device=dev)
                      .to(torch.bfloat16) for _ in range(3))
        qtp, ktp, vtp = (torch.empty((w.B, lpadp, w.H, w.D), dtype=torch.bfloat16, device=dev)
                         for _ in range(3))
        op = torch.empty_like(qp)
        bsta.attn_tile(gp, qp, out=qtp)
        bsta.attn_tile(gp, kp, out=ktp)
        selp = bsta.attn_select_packed(gp, qtp, ktp, 0.9, 0.5, want_mask=False)
        pqp, pkp = selp.pooled(gp)
        perp = {"tile_qkv": [], "select": [], "attn_fwd": []}
        for it in range(n_calls + 2):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            e[0].record()
            bsta.attn_tile_pool(gp, qp, pqp, out=qtp)
            bsta.attn_tile_pool(gp, kp, pkp, out=ktp)
            bsta.attn_tile(gp, vp, out=vtp)
            e[1].record()
            bsta.attn_select_packed(gp, None, None, 0.9, 0.5, prepooled=True, out=selp)
            e[2].record()
            bsta.attn_block_sparse_fwd(gp, qtp, ktp, vtp, selp.row_ptr, selp.col_idx, out=op,
                                       raster=True)
            e[3].record()
            torch.cuda.synchronize()
            if it >= 2:
                for idx, n in enumerate(perp):
                    perp[n].append(e[idx].elapsed_time(e[idx + 1]))
        nnzp = int(selp.row_ptr[-1].item())
        msp = {n: float(np.median(v_)) for n, v_ in perp.items()}
        flopp = attention_flop(w, nnzp)
        packed_leg = {"segments": [226, [4, w.Y, w.X], [w.T, w.Y, w.X]], "tiles": ntp,
                      "prefix_tiles": info["num_prefix"], "spans": info["spans"],
                      "packed_len": info["L"], "sparsity": 0.9, "ref_keep_rate": 0.5,
                      "selected_tile_pairs": nnzp, "tile_qkv_ms": msp["tile_qkv"],
                      "select_ms": msp["select"], "attn_ms": msp["attn_fwd"],
                      "attn_tflops": flopp / (msp["attn_fwd"] * 1e-3) / 1e12,
                      "attn_frac_mfma_peak": flopp / (msp["attn_fwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                      "note": "packed sequence: tile_pool/tile, exempt selection from pooled "
                              "(prefix kept whole, per-region top-k), raster attention; "
                              "not in the step"}
        print(f"[bench] packed sequence {packed_leg}", file=sys.stderr, flush=True)
        del qp, kp, vp, qtp, ktp, vtp, op, selp

    # The backward (attn_block_sparse_bwd) on the step's selection, with a
    # seeded synthetic output gradient; not part of the step.  Its
    # algorithmic work is five products per selected pair (S, dP, dV, dQ,
    # dK), 2.5 times the forward's two.
    bwd = None
    if bwd_leg and nt <= 4096:
        _, lse_b = bsta.attn_block_sparse_fwd(g, qt, kt, vt, sel.row_ptr, sel.col_idx, out=ot,
                                              want_lse=True)
        gen = torch.Generator(device=dev).manual_seed(7)
        dot_b = torch.randn((w.B, lpad, w.H, w.D), generator=gen, device=dev).to(torch.bfloat16)
        grads = tuple(torch.empty_like(qt) for _ in range(3))
        bsta.attn_block_sparse_bwd(g, qt, kt, vt, ot, dot_b, lse_b, sel.row_ptr, sel.col_idx,
                                   out=grads)
        per_b = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            bsta.attn_block_sparse_bwd(g, qt, kt, vt, ot, dot_b, lse_b, sel.row_ptr, sel.col_idx,
                                       out=grads)
            e1.record()
            torch.cuda.synchronize()
            per_b.append(e0.elapsed_time(e1))
        b_ms = float(np.median(per_b))
        b_flop = 2.5 * attention_flop(w, nnz)
        bwd = {"ms": b_ms, "tflops": b_flop / (b_ms * 1e-3) / 1e12,
               "frac_mfma_peak": b_flop / (b_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
               "algorithmic_flop": b_flop, "calls": 5, "stat": "median",
               "note": "attn_block_sparse_bwd (delta, CSR transpose, dQ, dK/dV) on the step's "
                       "selection; not in the step"}
        print(f"[bench] backward {bwd}", file=sys.stderr, flush=True)
        del grads, dot_b, lse_b

    flop = attention_flop(w, nnz)
    prof = measured_attn() if args.workload == "c3" and not args.deterministic else None
    dense_flop = 4.0 * w.D * w.B * w.H * float(w.L) ** 2
    attn_tflops = flop / (ms["attn_fwd"] * 1e-3) / 1e12
    elem = w.B * w.H * w.D * 2
    pooled_bytes = 2 * w.B * w.H * nt * w.D * 4 if fused else 0
    tile_bytes = 3 * elem * (w.L + lpad) + pooled_bytes
    tile_qk_bytes = 2 * elem * (w.L + lpad) + pooled_bytes
    tile_v_bytes = elem * (w.L + lpad)
    untile_bytes = elem * (w.L + lpad)
    pool_bytes = 2 * elem * w.L + 2 * w.B * w.H * nt * w.D * 4
    out = {
        "metric": METRIC,
        "value": flop / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: B={w.B} H={w.H} D={w.D} grid {w.T}x{w.Y}x{w.X} "
                        f"(L={w.L}, {nt} tiles of 4x4x4), "
                        + (f"top-k {w.topk}" if w.mode == "topk" else "STA windows"),
            "selected_tile_pairs": nnz,
            "attn_key_order": "csr order (deterministic)" if args.deterministic
                              else "rotated walk (library default)",
            "value_basis": "selected-tile attention FLOP (4*D*64*64 per pair) per whole-path step",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_fwd_kernel<128, 1>",
            "achieved": attn_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": attn_tflops / PEAK_BF16_TFLOPS,
            "traffic": prof["traffic_bytes"] if prof else None,
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE/WRITE_SIZE, copy-calibrated)",
            "algorithmic_flop_per_launch": flop,
            "counters": ({k: prof[k] for k in ("l2_hit", "lds_bank_conflict_per_active",
                                               "mfma_busy", "clock_ghz",
                                               "insts_per_key_tile_wave")} if prof else None),
        },
        "kernels": {
            "attn_fwd": {"ms": ms["attn_fwd"], "tflops": attn_tflops,
                         "dense_equiv_tflops": dense_flop / (ms["attn_fwd"] * 1e-3) / 1e12,
                         "valid_token_flop": valid_flop,
                         "valid_token_tflops": valid_flop / (ms["attn_fwd"] * 1e-3) / 1e12,
                         "frac_mfma_peak": attn_tflops / PEAK_BF16_TFLOPS,
                         "calls": n_calls, "stat": "median",
                         "note": "attn_block_sparse_fwd_raster (output in raster order)"},
            "attn_fwd_cold_l2": ({"ms": cold_ms, "tflops": flop / (cold_ms * 1e-3) / 1e12,
                                  "frac_mfma_peak": flop / (cold_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                  "note": "512 MB write before each call"} if cold_ms else None),
            "tile_qkv": {"ms": ms["tile_qkv"], "gbps": tile_bytes / (ms["tile_qkv"] * 1e-3) / 1e9,
                         "frac_hbm_peak": tile_bytes / (ms["tile_qkv"] * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                         "note": ("attn_tile_pool for Q and K (pooling fused), attn_tile for V"
                                  if fused else "attn_tile for Q, K and V")},
            "tile_pool": {"ms": ms["tile_qk"], "bytes": tile_qk_bytes,
                          "gbps": tile_qk_bytes / (ms["tile_qk"] * 1e-3) / 1e9,
                          "frac_hbm_peak": tile_qk_bytes / (ms["tile_qk"] * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                          "note": ("attn_tile_pool for Q and K: read L rows, write Lpad rows and the "
                                   "pooled vectors, per tensor" if fused else "attn_tile for Q and K")},
            "tile_v": {"ms": ms["tile_v"], "gbps": tile_v_bytes / (ms["tile_v"] * 1e-3) / 1e9,
                       "frac_hbm_peak": tile_v_bytes / (ms["tile_v"] * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                       "note": "attn_tile for V"},
            "pool": {"ms": pool_ms, "bytes": pool_bytes,
                     "gbps": pool_bytes / (pool_ms * 1e-3) / 1e9,
                     "frac_hbm_peak": pool_bytes / (pool_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                     "note": "attn_pool on the tiled Q and K (the pooling step alone: read the valid "
                             "rows, write the pooled vectors); not in the step"},
            "select": {"ms": ms["select"],
                       "note": "scores + top-k (prepooled)" if fused else "window CSR"},
            "select_unfused": ({"ms": unfused_ms, "pool_bytes": pool_bytes,
                                "note": "pool + scores + top-k from the tiled Q and K; not in the step"}
                               if fused else None),
            "untile": ({"ms": untile_ms, "gbps": untile_bytes / (untile_ms * 1e-3) / 1e9,
                        "note": "standalone attn_untile; not in the step (attn_fwd writes raster order)"}
                       if untile_ms else None),
            "select_cumulative": cum,
            "pruned_queries": pruned,
            "tile128": t128,
            "packed": packed_leg,
            "attn_bwd": bwd,
        },
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
