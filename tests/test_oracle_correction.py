"""Pins for the oracle's output correction (SSDi8's per-channel mean correction) and for the
recurrence over real-valued inputs that the correction is calibrated against (CPU only).

The pages name the correction (the SSDi8 abstract describes a correction derived from error
statistics gathered per channel; Figure 1b labels it a mean correction; ablated in Table 6, timed
in Table 16) but give
neither its algebra nor any value, so nothing here is pinned by a printed number; the reading
(an additive per-(head, channel) term, calibrated as the mean over a calibration draw of the
unquantized scan's y minus the quantized scan's y) is pinned by exact identities instead:
  - the real-valued recurrence against the independent numpy chunked dual form;
  - y with the correction minus y without it is the correction, broadcast over (batch, token);
  - inputs that are exactly their dequantized codes calibrate to a zero correction;
  - inputs offset from their codes by exactly a quarter step calibrate to the scan's response
    to that constant offset, computed independently by linearity with the chunked form;
  - after correction the calibration draw's mean error per channel vanishes."""
import math

import numpy as np

import oracle
from ref_chunked import chunked_ssd


def _params(seed, H=4, G=2, b=2, L=40):
    rng = np.random.default_rng(seed)
    dt = np.log1p(np.exp(rng.normal(-2, 0.5, size=(b, L, H)))).astype(np.float32)
    A = (-np.exp(rng.uniform(0, math.log(16), size=H))).astype(np.float32)
    D = rng.uniform(0.5, 1.5, size=H).astype(np.float32)
    return rng, dt, A, D


def test_real_valued_recurrence_matches_the_chunked_dual_form():
    rng, dt, A, D = _params(1)
    b, L, H, P, N, G = 2, 40, 4, 3, 5, 2
    x = rng.normal(size=(b, L, H, P))
    B = rng.normal(size=(b, L, G, N))
    C = rng.normal(size=(b, L, G, N))
    h0 = rng.normal(0, 0.1, size=(b, H, P, N)).astype(np.float32)
    ones = lambda n: np.ones(n, np.float32)
    ref = chunked_ssd(x, ones(H), B, ones(G), C, ones(G), dt, A, D, h0, chunk=16)
    v = dict(x=x, B=B, C=C, dt=dt, A=A, D=D, h0=h0)
    for bb in range(b):
        for h in range(H):
            y, hf = oracle.ssd_values_one(v, bb, h)
            assert np.max(np.abs(y - ref["y"][bb, :, h])) <= 1e-12 * np.max(np.abs(ref["y"]))
            assert np.max(np.abs(hf - ref["h_final"][bb, h])) <= 1e-12 * np.max(np.abs(ref["h_final"]))


def _codes(seed, b=2, L=40, H=4, P=3, N=5, G=2, y_corr=None):
    rng, dt, A, D = _params(seed, H, G, b, L)
    qx = rng.integers(-127, 128, size=(b, L, H, P), dtype=np.int8)
    qB = rng.integers(-127, 128, size=(b, L, G, N), dtype=np.int8)
    qC = rng.integers(-127, 128, size=(b, L, G, N), dtype=np.int8)
    sx = rng.uniform(0.005, 0.05, size=H).astype(np.float32)
    sB = rng.uniform(0.005, 0.05, size=G).astype(np.float32)
    sC = rng.uniform(0.005, 0.05, size=G).astype(np.float32)
    return oracle.Codes(qx, sx, qB, sB, qC, sC, dt, A, D, None, y_corr)


def test_correction_is_added_to_every_output():
    H, P = 4, 3
    mu = np.random.default_rng(2).normal(size=(H, P)).astype(np.float32)   # H != P: a transposed index shows
    c0 = _codes(3)
    c1 = _codes(3, y_corr=mu)
    cz = _codes(3, y_corr=np.zeros((H, P), np.float32))
    y0, h0, _ = oracle.ssd(c0, threads=1)
    y1, h1, _ = oracle.ssd(c1, threads=1)
    yz, _, _ = oracle.ssd(cz, threads=1)
    assert np.array_equal(y0, yz)
    assert np.array_equal(h0, h1)                                   # the state is not touched
    assert np.max(np.abs((y1 - y0) - mu[None, None].astype(np.float64))) <= 1e-13 * np.max(np.abs(y0))
    # the cached-state recurrences carry it the same way
    y16, _, _ = oracle.ssd_one(c1, 1, 2, state_f16=True)
    y16_0, _, _ = oracle.ssd_one(c0, 1, 2, state_f16=True)
    assert np.max(np.abs(y16 - y16_0 - mu[2].astype(np.float64))) <= 1e-13 * np.max(np.abs(y16_0))
    y8, *_ = oracle.ssd_one_state_i8(c1, 1, 2)
    y8_0, *_ = oracle.ssd_one_state_i8(c0, 1, 2)
    assert np.max(np.abs(y8 - y8_0 - mu[2].astype(np.float64))) <= 1e-13 * np.max(np.abs(y8_0))


def _draw(seed, offset, b=2, L=48, H=4, P=8, N=8, G=2):
    """Binary16 activations that are exactly s * (code + offset), with power-of-two scales so that
    every value is a binary16 number; the codes are then exactly `code`."""
    rng, dt, A, D = _params(seed, H, G, b, L)
    sx = np.exp2(rng.integers(-7, -3, size=H)).astype(np.float32)
    sB = np.exp2(rng.integers(-7, -3, size=G)).astype(np.float32)
    sC = np.exp2(rng.integers(-7, -3, size=G)).astype(np.float32)
    qx = rng.integers(-120, 121, size=(b, L, H, P))
    qB = rng.integers(-120, 121, size=(b, L, G, N))
    qC = rng.integers(-120, 121, size=(b, L, G, N))
    x16 = ((qx + offset) * sx[:, None]).astype(np.float16)
    assert np.array_equal(x16.astype(np.float64), (qx + offset) * sx[:, None].astype(np.float64))
    return dict(x16=x16, B16=(qB * sB[:, None]).astype(np.float16), C16=(qC * sC[:, None]).astype(np.float16),
                x_scale=sx, B_scale=sB, C_scale=sC, dt=dt, A=A, D=D,
                h0=rng.normal(0, 0.1, size=(b, H, P, N)).astype(np.float32)), qx


def test_exact_codes_calibrate_to_zero():
    inp, _ = _draw(4, 0.0)
    assert np.all(oracle.mean_correction(inp, threads=2) == 0)


def test_quarter_step_offset_calibrates_to_the_response_to_that_offset():
    # x16 = s_x (q + 1/4): the codes are q, so the unquantized scan differs from the quantized one
    # by the (linear) scan of the constant input s_x / 4 alone, with B, C exact and no h0
    inp, qx = _draw(5, 0.25)
    c = oracle.codes_from_inputs(inp)
    assert np.array_equal(c.qx, qx.astype(np.int8))
    mu = oracle.mean_correction(inp, threads=2)
    b, L, H, P = inp["x16"].shape
    quarter = np.full((b, L, H, P), 0.25)
    resp = chunked_ssd(quarter, inp["x_scale"], c.qB, c.sB, c.qC, c.sC, c.dt, c.A, c.D, None, chunk=L)["y"]
    want = resp.mean(axis=(0, 1))                                   # (H, P)
    assert np.max(np.abs(mu - want)) <= 1e-6 * np.max(np.abs(want)) + 1e-12
    assert np.max(np.abs(want)) > 0


def test_corrected_calibration_error_has_zero_mean():
    rng = np.random.default_rng(6)
    inp, _ = _draw(6, 0.0)
    # generic binary16 values (not exact codes) with absmax/127 scales
    b, L, H, P = inp["x16"].shape
    x = rng.normal(0.5, 1.0, size=(b, L, H, P)).astype(np.float16)
    inp["x16"] = x
    inp["x_scale"] = (np.abs(x.astype(np.float32)).max(axis=(0, 1, 3)) / np.float32(127)).astype(np.float32)
    mu = oracle.mean_correction(inp, threads=2)
    c = oracle.codes_from_inputs(dict(inp, y_corr=mu))
    vals = dict(x=inp["x16"].astype(np.float64), B=inp["B16"].astype(np.float64), C=inp["C16"].astype(np.float64),
                dt=inp["dt"], A=inp["A"], D=inp["D"], h0=inp["h0"])
    err = np.zeros((H, P))
    scale = 0.0
    for bb in range(b):
        for h in range(H):
            y_ref, _ = oracle.ssd_values_one(vals, bb, h)
            y_c, _, _ = oracle.ssd_one(c, bb, h)
            err[h] += (y_ref - y_c).sum(axis=0)
            scale = max(scale, np.max(np.abs(y_ref)))
    # what is left is the float32 rounding of mu
    assert np.max(np.abs(err / (b * L))) <= 1e-6 * max(np.max(np.abs(mu)), 1e-30) + 1e-12 * scale
