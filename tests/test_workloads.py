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


def test_percentile_scale_clips_at_the_quantile():
    rng = np.random.default_rng(3)
    t = rng.normal(size=(5000, 2, 8)).astype(np.float16)
    s = workloads.percentile_scale(t, -2, 99.0)
    a = np.abs(t.astype(np.float32))
    for h in range(2):
        q = np.float32(np.percentile(a[:, h, :], 99.0))
        assert s[h] == q / np.float32(127)
        assert np.mean(a[:, h, :] > q) <= 0.011              # about 1% saturates
    assert np.all(workloads.percentile_scale(np.zeros((4, 2, 8), np.float16), -2, 99.0) == 1)


def test_calibrated_pair_shares_model_and_scales():
    shape = workloads.PrefillShape("pair", 2, 64, 4, 16, 32, 2, 64, "outlier_heads", "fixed_bias", 0.1)
    cal, test = workloads.make_calibrated_pair(shape, 60, x_mean=0.5, x_clip_pct=99.0)
    for k in ("A", "D", "x_scale", "B_scale", "C_scale"):
        assert np.array_equal(cal[k], test[k])
    assert not np.array_equal(cal["x16"], test["x16"]) and cal["h0"] is not None
    assert np.array_equal(cal["x_scale"], workloads.percentile_scale(cal["x16"], -2, 99.0))
    # x = m_h (N(0, 1) + 0.5): one-sided on average
    assert np.mean(test["x16"].astype(np.float32)) > 0.2


def test_per_state_scales():
    shape = workloads.PrefillShape("pn", 2, 64, 4, 16, 32, 2, 64, "normal", "fixed_bias", 0.0)
    cal, test = workloads.make_calibrated_pair(shape, 61, bc_per_state=True, state_spread=1.0)
    assert cal["B_scale"].shape == (2, 32) and test["C_scale"].shape == (2, 32)
    amax = np.abs(cal["B16"].astype(np.float32)).max(axis=(0, 1))
    assert np.array_equal(cal["B_scale"], (amax / np.float32(127)).astype(np.float32))
    # the state columns carry their own magnitudes: the scales spread well beyond one group's
    assert cal["B_scale"].max() / cal["B_scale"].min() > 4


def test_cluster_channel_scales():
    rng = np.random.default_rng(5)
    x = (rng.normal(size=(64, 3, 8)) * np.exp(rng.normal(size=(3, 8)))).astype(np.float16)
    amax = np.abs(x.astype(np.float32)).max(axis=0)
    # one cluster: the per-head absmax scale on every channel; P clusters: one per channel
    one = workloads.cluster_channel_scales(x, 1)
    assert np.array_equal(one, np.repeat(workloads.absmax_scale(x, -2)[:, None], 8, axis=1))
    assert np.array_equal(workloads.cluster_channel_scales(x, 8), (amax / np.float32(127)).astype(np.float32))
    # k clusters: k distinct scales per head, each the largest absmax of its members, and the
    # clusters are runs of the channels sorted by absmax
    for k in (2, 3):
        s = workloads.cluster_channel_scales(x, k)
        assert s.shape == (3, 8) and s.dtype == np.float32
        for h in range(3):
            assert len(np.unique(s[h])) == k
            assert np.all(s[h] * 127 >= amax[h] * (1 - 1e-6))
            order = np.argsort(amax[h], kind="stable")
            assert np.all(np.diff(s[h][order]) >= 0)
            for v in np.unique(s[h]):
                assert np.isclose(v * 127, amax[h][s[h] == v].max(), rtol=1e-6)
