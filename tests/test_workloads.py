"""Host-side checks of the seeded workload generators (CPU only)."""
import numpy as np

import workloads


def test_tiny_shapes_and_determinism():
    a = workloads.make_prefill("tiny")
    b = workloads.make_prefill("tiny")
    assert a["x16"].shape == (1, 256, 4, 16) and a["x16"].dtype == np.float16
    assert a["B16"].shape == (1, 256, 1, 16) and a["C16"].shape == (1, 256, 1, 16)
    assert a["dt"].shape == (1, 256, 4) and a["dt"].dtype == np.float32
    for k in ("x16", "B16", "C16", "dt", "A", "D", "x_scale", "B_scale", "C_scale"):
        assert np.array_equal(a[k], b[k])
    assert a["h0"] is None


def test_parameter_ranges():
    a = workloads.make_prefill("tiny")
    assert np.all(a["A"] <= -1.0) and np.all(a["A"] >= -16.0)
    assert np.all(a["D"] >= 0.5) and np.all(a["D"] <= 1.5)
    assert np.all(a["dt"] > 0)
    for s in (a["x_scale"], a["B_scale"], a["C_scale"]):
        assert s.dtype == np.float32 and np.all(s > 0)


def test_scales_come_from_a_separate_calibration_draw():
    a = workloads.make_prefill("tiny")
    # absmax of the test draw differs from the calibration absmax (separate seeds)
    test_absmax = np.abs(a["x16"].astype(np.float32)).max(axis=(0, 1, 3)) / np.float32(127)
    assert not np.array_equal(test_absmax.astype(np.float32), a["x_scale"])


def test_outlier_heads_share_model_seed():
    shape = workloads.WORKLOADS["mamba2-1.3b-prefill"]
    p = workloads.model_params(shape.nheads, shape.x_dist, shape.dt_dist, 101)
    assert np.sum(p.x_mag == 20.0) == round(0.1 * 64)
    a = workloads.make_prefill("mamba2-1.3b-prefill", batch=1, seqlen=64)
    big = a["x_scale"] > 5 * np.median(a["x_scale"])
    assert np.array_equal(big, p.x_mag == 20.0)


def test_decode_shapes():
    d = workloads.make_decode("mamba2-8b-decode", batch=2, steps=3)
    assert d["state"].shape == (2, 128, 64, 128)
    assert d["x16"].shape == (3, 2, 128, 64)
    assert d["B16"].shape == (3, 2, 8, 128)
    assert d["dt"].shape == (3, 2, 128)
