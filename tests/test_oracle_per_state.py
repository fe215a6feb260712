"""Pins for the oracle with B and C scales per (group, state) (SSDi8 Table 10's per-P(N) axis
together with per-H(G)) (CPU only):
  - the per-(k, i) quantizer against the pinned per-k quantizer applied column by column;
  - constant scales along the states reproduce the per-group oracle exactly;
  - the recurrence over the codes equals the real-valued recurrence over the same dequantized
    values (exactly) and the independent numpy chunked dual form;
  - the chunk state obeys the chunk-boundary identity with per-state scales."""
import math

import numpy as np

import oracle
from ref_chunked import chunked_ssd


def _codes(seed, per_state=True, b=2, L=37, H=4, P=3, N=5, G=2, h0=True):
    rng = np.random.default_rng(seed)
    qx = rng.integers(-127, 128, size=(b, L, H, P), dtype=np.int8)
    qB = rng.integers(-127, 128, size=(b, L, G, N), dtype=np.int8)
    qC = rng.integers(-127, 128, size=(b, L, G, N), dtype=np.int8)
    sx = rng.uniform(0.005, 0.05, size=H).astype(np.float32)
    shape = (G, N) if per_state else (G,)
    sB = rng.uniform(0.005, 0.05, size=shape).astype(np.float32)
    sC = rng.uniform(0.005, 0.05, size=shape).astype(np.float32)
    dt = np.log1p(np.exp(rng.normal(-2, 0.5, size=(b, L, H)))).astype(np.float32)
    A = (-np.exp(rng.uniform(0, math.log(16), size=H))).astype(np.float32)
    D = rng.uniform(0.5, 1.5, size=H).astype(np.float32)
    hh = rng.normal(0, 0.1, size=(b, H, P, N)).astype(np.float32) if h0 else None
    return oracle.Codes(qx, sx, qB, sB, qC, sC, dt, A, D, hh)


def test_per_channel_quantizer_is_the_per_k_quantizer_column_by_column():
    rng = np.random.default_rng(1)
    x = (rng.normal(size=(50, 3, 7)) * 4).astype(np.float16)
    x[0, 0, :3] = [np.inf, -np.inf, np.nan]
    s = rng.uniform(0.01, 0.2, size=(3, 7)).astype(np.float32)
    q = oracle.quantize_per_channel(x, s)
    for i in range(7):
        col = np.ascontiguousarray(x[:, :, i:i + 1])
        assert np.array_equal(q[:, :, i:i + 1], oracle.quantize(col, s[:, i]))
    flat = np.repeat(s[:, :1], 7, axis=1)
    assert np.array_equal(oracle.quantize_per_channel(x, flat), oracle.quantize(x, s[:, 0]))


def test_constant_state_scales_reproduce_the_per_group_oracle():
    c = _codes(2, per_state=False)
    cs = _codes(2, per_state=False)
    cs.sB = np.repeat(c.sB[:, None], c.N, axis=1)
    cs.sC = np.repeat(c.sC[:, None], c.N, axis=1)
    cs.per_state = 1
    y, h, bounds = oracle.ssd(c, chunk=8, threads=1)
    ys, hs, bs = oracle.ssd(cs, chunk=8, threads=1)
    assert np.array_equal(y, ys) and np.array_equal(h, hs) and np.array_equal(bounds, bs)
    assert np.array_equal(oracle.chunk_state(c, 1, 2, 8), oracle.chunk_state(cs, 1, 2, 8))
    y8, *_ = oracle.ssd_one_state_i8(c, 1, 3)
    y8s, *_ = oracle.ssd_one_state_i8(cs, 1, 3)
    assert np.array_equal(y8, y8s)


def _dequantized(c):
    x = c.qx.astype(np.float64) * c.sx.astype(np.float64)[:, None]
    B = c.qB.astype(np.float64) * c.sB.astype(np.float64)
    C = c.qC.astype(np.float64) * c.sC.astype(np.float64)
    return x, B, C


def test_per_state_recurrence_is_the_recurrence_over_its_dequantized_values():
    c = _codes(3)
    x, B, C = _dequantized(c)
    v = dict(x=x, B=B, C=C, dt=c.dt, A=c.A, D=c.D, h0=c.h0)
    y, hf, _ = oracle.ssd(c, threads=1)
    for b in range(c.batch):
        for h in range(c.H):
            yv, hv = oracle.ssd_values_one(v, b, h)
            assert np.array_equal(y[b, :, h], yv) and np.array_equal(hf[b, h], hv)
    ones = lambda n: np.ones(n, np.float32)
    ref = chunked_ssd(x, ones(c.H), B, ones(c.G), C, ones(c.G), c.dt, c.A, c.D, c.h0, chunk=16)
    assert np.max(np.abs(y - ref["y"])) <= 1e-12 * np.max(np.abs(ref["y"]))
    assert np.max(np.abs(hf - ref["h_final"])) <= 1e-12 * np.max(np.abs(ref["h_final"]))


def test_per_state_chunk_state_links_boundary_states():
    c = _codes(4, L=40)
    _, _, bounds = oracle.ssd(c, chunk=8, threads=1)
    hf = oracle.ssd(c, threads=1)[1]
    for b in range(c.batch):
        for h in range(c.H):
            S = oracle.chunk_state(c, b, h, 8)
            acs = oracle.chunk_cumsum(c, b, h, 8)
            nxt = np.concatenate([bounds[b, 1:, h], hf[b, h][None]])
            pred = np.exp(acs[:, -1])[:, None, None] * bounds[b, :, h] + S
            assert np.max(np.abs(pred - nxt)) <= 1e-12 * np.max(np.abs(nxt))
