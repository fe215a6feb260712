"""Pins for the oracle's front end (depthwise causal conv1d + bias + SiLU, rounded to binary16,
then the static quantizer) and for dt = softplus(dt_raw + dt_bias).

The convolution is checked against numpy's own full convolution per channel (a library routine;
a flipped kernel, a shifted tap or a missing zero history fails it) and for causality; SiLU by
its identities (SiLU(v) - SiLU(-v) = v, SiLU(0) = 0, SiLU(ln 3) = (3/4) ln 3) and its limits;
the binary16 rounding against numpy's float16 conversion; the codes against the already pinned
quantizer applied to that binary16 output; softplus by its identities (softplus(v) -
softplus(-v) = v, softplus(0) = ln 2) and against numpy's logaddexp."""
import math

import numpy as np

import oracle

H, P, G, N = 2, 16, 1, 16
C = H * P + 2 * G * N


def _draw(rng, b=2, L=23, dconv=4, std=2.0):
    x = (rng.standard_normal((b, L, C)) * std).astype(np.float16)
    w = (rng.standard_normal((C, dconv)) * 0.5).astype(np.float16).astype(np.float32)
    bias = (rng.standard_normal(C) * 0.1).astype(np.float16).astype(np.float32)
    scales = [rng.uniform(0.01, 0.05, n).astype(np.float32) for n in (H, G, G)]
    return x, w, bias, scales


def test_convolution_matches_numpy_per_channel():
    rng = np.random.default_rng(21)
    x, w, bias, (sx, sB, sC) = _draw(rng)
    out = oracle.frontend(x, w, bias, sx, sB, sC, H, P, G, N)
    b, L, _ = x.shape
    for bi in range(b):
        for ch in range(C):
            # tap k multiplies token t - 3 + k: a true convolution with the reversed taps
            full = np.convolve(x[bi, :, ch].astype(np.float64), w[ch, ::-1].astype(np.float64))
            assert np.allclose(out["pre"][bi, :, ch], full[:L] + bias[ch], rtol=1e-13, atol=1e-13)


def test_causality_and_reach():
    """A change at token t0 moves the outputs of tokens t0 .. t0 + 3 only."""
    rng = np.random.default_rng(22)
    x, w, bias, (sx, sB, sC) = _draw(rng, b=1, L=16)
    base = oracle.frontend(x, w, bias, sx, sB, sC, H, P, G, N)["pre"]
    x2 = x.copy()
    x2[0, 6] += np.float16(1.0)
    moved = np.any(oracle.frontend(x2, w, bias, sx, sB, sC, H, P, G, N)["pre"] != base, axis=2)[0]
    assert list(np.nonzero(moved)[0]) == [6, 7, 8, 9]


def test_silu_identities_and_limits():
    rng = np.random.default_rng(23)
    L = 9
    v = np.concatenate([[0.0, math.log(3.0), 30.0, -30.0], rng.uniform(-8, 8, L - 4)])
    ident = np.zeros((C, 4), np.float32)
    ident[:, 3] = 1.0                                     # output = SiLU(input of the same token)
    x = np.zeros((1, L, C), np.float16)
    x[0, :, 0] = v.astype(np.float16)
    x[0, :, 1] = (-v).astype(np.float16)
    one = np.ones(H, np.float32), np.ones(G, np.float32), np.ones(G, np.float32)
    out = oracle.frontend(x, ident, None, *one, H, P, G, N)
    vv = x[0, :, 0].astype(np.float64)
    a, a_neg = out["act"][0, :, 0], out["act"][0, :, 1]
    assert np.allclose(a - a_neg, vv, rtol=1e-15, atol=1e-15)          # SiLU(v) - SiLU(-v) = v
    assert a[0] == 0.0
    # SiLU(ln 3) = (3/4) ln 3; the input is ln 3 rounded to binary16, and near ln 3 the slope of
    # SiLU(v) - (3/4) v is about 0.21, so the offset is at most a quarter of the input's error
    assert abs(a[1] - 0.75 * vv[1]) <= 1e-15 + 0.25 * abs(vv[1] - math.log(3.0))
    assert out["act16"][0, 2, 0] == np.float16(30.0) and out["act16"][0, 3, 0] == 0.0
    assert np.all(a[4:] > np.minimum(vv[4:], 0) - 0.2785)              # SiLU >= its minimum -0.2785
    # zero history: the first token sees only its own input
    out2 = oracle.frontend(np.ones((1, 3, C), np.float16), np.ones((C, 4), np.float32), None, *one, H, P, G, N)
    assert np.array_equal(out2["pre"][0, :, 0], [1.0, 2.0, 3.0])


def test_binary16_output_and_codes():
    rng = np.random.default_rng(24)
    x, w, bias, (sx, sB, sC) = _draw(rng, std=4.0)
    out = oracle.frontend(x, w, bias, sx, sB, sC, H, P, G, N)
    assert np.array_equal(out["act16"], out["act"].astype(np.float16))   # numpy's own rounding
    a16 = out["act16"]
    hp, gn = H * P, G * N
    b, L, _ = x.shape
    assert np.array_equal(out["qx"], oracle.quantize(a16[..., :hp].reshape(b, L, H, P), sx))
    assert np.array_equal(out["qB"], oracle.quantize(a16[..., hp:hp + gn].reshape(b, L, G, N), sB))
    assert np.array_equal(out["qC"], oracle.quantize(a16[..., hp + gn:].reshape(b, L, G, N), sC))


def test_softplus():
    rng = np.random.default_rng(25)
    raw = rng.uniform(-30, 30, (50, 4)).astype(np.float32)
    bias = rng.uniform(-2, 2, 4).astype(np.float32)
    sp = oracle.softplus_dt(raw, bias)
    v = raw.astype(np.float64) + bias
    assert np.allclose(sp, np.logaddexp(0.0, v), rtol=1e-15, atol=0)
    neg = oracle.softplus_dt(-raw, -bias)
    assert np.allclose(sp - neg, v, rtol=0, atol=1e-13)                  # softplus(v) - softplus(-v) = v
    assert oracle.softplus_dt(np.zeros((1, 1), np.float32), None)[0, 0] == math.log(2.0)
    big = oracle.softplus_dt(np.array([[100.0, -100.0]], np.float32), None)[0]
    assert big[0] == 100.0 and 0 < big[1] < 1e-43
