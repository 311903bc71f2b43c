"""The seeded input generators: determinism, shapes, bf16 rounding."""
import numpy as np
import torch

import workloads


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, -3.3e-5], np.float32)])
    ours = workloads.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(workloads.bf16_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_small_workload_deterministic():
    w = workloads.WORKLOADS["c1"]
    a = workloads.make_inputs(w)
    b = workloads.make_inputs(w)
    for key in ("q", "k", "v"):
        assert a[key].shape == (w.B, w.L, w.H, w.D) and a[key].dtype == np.uint16
        assert np.array_equal(a[key], b[key])
    assert not np.array_equal(a["q"], a["k"])


def test_structured_workloads_small():
    w = workloads.custom("lr", 1, 2, 16, 8, 8, 12, structure="lowrank", seed=5)
    x = workloads.make_inputs(w)
    q = workloads.bf16_to_f32(x["q"])
    assert abs(q.std() - np.sqrt(1.25)) < 0.1
    w2 = workloads.custom("sm", 1, 1, 8, 8, 12, 12, structure="smooth", seed=5)
    assert workloads.make_inputs(w2)["k"].shape == (1, 8 * 12 * 12, 1, 8)


def test_sta_windows():
    w = workloads.WORKLOADS["c5"]
    win = workloads.sta_windows(w)
    assert win.shape == (24, 3)
    assert {tuple(r) for r in win} <= set(workloads.STA_CANDIDATES)
    assert np.array_equal(win, workloads.sta_windows(w))
