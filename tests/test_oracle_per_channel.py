"""Pins for the oracle with x scales per (head, channel) -- the static scales that Quamba2's
sort-and-cluster of channels leaves behind, one per channel cluster, expanded here to every
channel (CPU only):
  - the quantizer of x under (H, P) scales is the per-head quantizer applied channel by channel;
  - constant channel scales reproduce the per-head oracle exactly (every state format);
  - channels are independent in the recurrence: channel p of every output under the (H, P) table
    equals the per-head oracle run with head h's scale set to s_x[h, p] (a transposed or dropped
    index fails it), for the fp32, binary16 and 8-bit cached states and the chunk states;
  - the recurrence over the codes equals the real-valued recurrence over the same dequantized
    values (exactly) and the independent numpy chunked dual form, also together with B and C
    scales per (group, state);
  - the chunk state obeys the chunk-boundary identity."""
import math

import numpy as np

import oracle
from ref_chunked import chunked_ssd


def _codes(seed, per_state=False, b=2, L=37, H=4, P=3, N=5, G=2, h0=True):
    rng = np.random.default_rng(seed)
    qx = rng.integers(-127, 128, size=(b, L, H, P), dtype=np.int8)
    qB = rng.integers(-127, 128, size=(b, L, G, N), dtype=np.int8)
    qC = rng.integers(-127, 128, size=(b, L, G, N), dtype=np.int8)
    sx = rng.uniform(0.005, 0.05, size=(H, P)).astype(np.float32)
    shape = (G, N) if per_state else (G,)
    sB = rng.uniform(0.005, 0.05, size=shape).astype(np.float32)
    sC = rng.uniform(0.005, 0.05, size=shape).astype(np.float32)
    dt = np.log1p(np.exp(rng.normal(-2, 0.5, size=(b, L, H)))).astype(np.float32)
    A = (-np.exp(rng.uniform(0, math.log(16), size=H))).astype(np.float32)
    D = rng.uniform(0.5, 1.5, size=H).astype(np.float32)
    hh = rng.normal(0, 0.1, size=(b, H, P, N)).astype(np.float32) if h0 else None
    return oracle.Codes(qx, sx, qB, sB, qC, sC, dt, A, D, hh)


def _per_head(c, sx_head):
    """The same codes with one x scale per head."""
    return oracle.Codes(c.qx, sx_head, c.qB, c.sB, c.qC, c.sC, c.dt, c.A, c.D, c.h0)


def test_x_codes_under_channel_scales_are_the_per_head_codes_channel_by_channel():
    rng = np.random.default_rng(1)
    inp = dict(x16=(rng.normal(size=(2, 9, 4, 3)) * 4).astype(np.float16),
               B16=(rng.normal(size=(2, 9, 2, 5))).astype(np.float16),
               C16=(rng.normal(size=(2, 9, 2, 5))).astype(np.float16),
               x_scale=rng.uniform(0.01, 0.2, size=(4, 3)).astype(np.float32),
               B_scale=np.full(2, 0.02, np.float32), C_scale=np.full(2, 0.02, np.float32),
               dt=np.full((2, 9, 4), 0.1, np.float32), A=-np.ones(4, np.float32))
    c = oracle.codes_from_inputs(inp)
    assert c.x_per_channel == 1 and c.scale_flags == 2
    for p in range(3):
        col = np.ascontiguousarray(inp["x16"][..., p:p + 1])
        assert np.array_equal(c.qx[..., p:p + 1], oracle.quantize(col, inp["x_scale"][:, p]))


def test_constant_channel_scales_reproduce_the_per_head_oracle():
    c = _codes(2)
    sx_head = c.sx[:, 0].copy()
    ch = _per_head(c, sx_head)
    cc = oracle.Codes(c.qx, np.repeat(sx_head[:, None], c.P, axis=1), c.qB, c.sB, c.qC, c.sC, c.dt, c.A, c.D, c.h0)
    y, h, bounds = oracle.ssd(ch, chunk=8, threads=1)
    yc, hc, bc = oracle.ssd(cc, chunk=8, threads=1)
    assert np.array_equal(y, yc) and np.array_equal(h, hc) and np.array_equal(bounds, bc)
    assert np.array_equal(oracle.chunk_state(ch, 1, 2, 8), oracle.chunk_state(cc, 1, 2, 8))
    yf, hf, _ = oracle.ssd_one(ch, 0, 1, state_f16=True)
    yfc, hfc, _ = oracle.ssd_one(cc, 0, 1, state_f16=True)
    assert np.array_equal(yf, yfc) and np.array_equal(hf, hfc)
    y8, *_ = oracle.ssd_one_state_i8(ch, 1, 3)
    y8c, *_ = oracle.ssd_one_state_i8(cc, 1, 3)
    assert np.array_equal(y8, y8c)


def test_channels_are_independent_under_channel_scales():
    c = _codes(3)
    y, hf, bounds = oracle.ssd(c, chunk=8, threads=1)
    for p in range(c.P):
        ch = _per_head(c, np.ascontiguousarray(c.sx[:, p]))
        yp, hp, bp = oracle.ssd(ch, chunk=8, threads=1)
        assert np.array_equal(y[..., p], yp[..., p])
        assert np.array_equal(hf[:, :, p], hp[:, :, p])
        assert np.array_equal(bounds[:, :, :, p], bp[:, :, :, p])
        assert np.array_equal(oracle.chunk_state(c, 1, 2, 8)[:, p], oracle.chunk_state(ch, 1, 2, 8)[:, p])
        yf, hff, _ = oracle.ssd_one(c, 1, 2, state_f16=True)
        yfp, hfp, _ = oracle.ssd_one(ch, 1, 2, state_f16=True)
        assert np.array_equal(yf[:, p], yfp[:, p]) and np.array_equal(hff[p], hfp[p])
        # the 8-bit cache re-quantizes each state row (one channel) on its own
        y8, h8, q8, s8, _ = oracle.ssd_one_state_i8(c, 0, 3)
        y8p, h8p, q8p, s8p, _ = oracle.ssd_one_state_i8(ch, 0, 3)
        assert np.array_equal(y8[:, p], y8p[:, p]) and np.array_equal(q8[p], q8p[p]) and s8[p] == s8p[p]


def _dequantized(c):
    x = c.qx.astype(np.float64) * c.sx.astype(np.float64)
    sB = c.sB.astype(np.float64) if c.per_state else c.sB.astype(np.float64)[:, None]
    sC = c.sC.astype(np.float64) if c.per_state else c.sC.astype(np.float64)[:, None]
    return x, c.qB.astype(np.float64) * sB, c.qC.astype(np.float64) * sC


def test_channel_scaled_recurrence_is_the_recurrence_over_its_dequantized_values():
    for per_state in (False, True):
        c = _codes(4, per_state=per_state)
        assert c.scale_flags == (3 if per_state else 2)
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


def test_channel_scaled_chunk_state_links_boundary_states():
    c = _codes(5, L=40, per_state=True)
    _, _, bounds = oracle.ssd(c, chunk=8, threads=1)
    hf = oracle.ssd(c, threads=1)[1]
    for b in range(c.batch):
        for h in range(c.H):
            S = oracle.chunk_state(c, b, h, 8)
            acs = oracle.chunk_cumsum(c, b, h, 8)
            nxt = np.concatenate([bounds[b, 1:, h], hf[b, h][None]])
            pred = np.exp(acs[:, -1])[:, None, None] * bounds[b, :, h] + S
            assert np.max(np.abs(pred - nxt)) <= 1e-12 * np.max(np.abs(nxt))
