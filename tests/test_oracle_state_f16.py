"""Pins for the oracle's binary16-cached state (the decode state kept in IEEE binary16 between
steps, a lower-precision cached state as the Quamba2 rebuttal's Tables R7/R8 discuss).

The rounding is checked against the IEEE binary16 format itself (every finite binary16 value
is a fixed point, midpoints go to the even neighbour, overflow goes to infinity) and against
numpy's independent float16 conversion; the recurrence is checked where the pages' arithmetic
fixes the answer (states exactly representable: no rounding at all), by brute force on one
token, and against the error bound that rounding once per step implies."""
import numpy as np

import oracle

ALL_F16 = np.arange(65536, dtype=np.uint16).view(np.float16)
FINITE = ALL_F16[np.isfinite(ALL_F16)].astype(np.float64)


def test_every_binary16_value_is_a_fixed_point():
    assert np.array_equal(oracle.round_binary16(FINITE), FINITE)


def test_midpoints_round_to_the_even_neighbour():
    pos = np.unique(FINITE[FINITE >= 0])                     # 0, subnormals, normals up to 65504
    lo, hi = pos[:-1], pos[1:]
    mid = (lo + hi) / 2                                     # exact in double
    got = oracle.round_binary16(mid)
    lo_bits = lo.astype(np.float16).view(np.uint16)
    want = np.where(lo_bits % 2 == 0, lo, hi)               # the neighbour with an even significand
    assert np.array_equal(got, want)
    assert np.array_equal(oracle.round_binary16(-mid), -want)
    # just off the midpoint: the nearer neighbour
    assert np.array_equal(oracle.round_binary16(np.nextafter(mid, lo)), lo)
    assert np.array_equal(oracle.round_binary16(np.nextafter(mid, hi)), hi)


def test_overflow_underflow_and_specials():
    r = oracle.round_binary16(np.array([65519.99, 65520.0, 1e9, -65520.0, 2.0 ** -25, 2.0 ** -25 * 1.0001,
                                        -(2.0 ** -26), 0.0, np.inf, np.nan]))
    assert r[0] == 65504.0 and r[1] == np.inf and r[2] == np.inf and r[3] == -np.inf
    assert r[4] == 0.0                     # exactly half the smallest subnormal: ties to even (0)
    assert r[5] == 2.0 ** -24              # just above it: the smallest subnormal
    assert r[6] == 0.0 and np.signbit(r[6])
    assert r[7] == 0.0 and r[8] == np.inf and np.isnan(r[9])


def test_random_doubles_match_numpys_conversion():
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
                        rng.uniform(-70000, 70000, 5000)])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).astype(np.float64)
    assert np.array_equal(oracle.round_binary16(v), ref)


def _codes(rng, T, H, P, N, G, dt_value=None, A_value=None, h0=None, small=False):
    qx = rng.integers(-3 if small else -127, 4 if small else 128, (1, T, H, P)).astype(np.int8)
    qB = rng.integers(-3 if small else -127, 4 if small else 128, (1, T, G, N)).astype(np.int8)
    qC = rng.integers(-127, 128, (1, T, G, N)).astype(np.int8)
    one = lambda n: np.ones(n, np.float32)
    sx, sB, sC = (one(H), one(G), one(G)) if small else (rng.uniform(0.01, 0.05, H).astype(np.float32),
                                                          rng.uniform(0.01, 0.05, G).astype(np.float32),
                                                          rng.uniform(0.01, 0.05, G).astype(np.float32))
    dt = np.full((1, T, H), dt_value, np.float32) if dt_value is not None else \
        rng.uniform(0.001, 0.1, (1, T, H)).astype(np.float32)
    A = np.full(H, A_value, np.float32) if A_value is not None else -rng.uniform(1, 16, H).astype(np.float32)
    D = rng.uniform(0.5, 1.5, H).astype(np.float32)
    return oracle.Codes(qx, sx, qB, sB, qC, sC, dt, A, D, h0)


def test_representable_states_are_not_rounded():
    """No decay (A = 0), dt = 1 and unit scales: every state is a sum of small integer products,
    exactly representable in binary16, so caching it changes nothing."""
    rng = np.random.default_rng(6)
    T, H, P, N, G = 40, 2, 4, 8, 1
    h0 = rng.integers(-50, 51, (1, H, P, N)).astype(np.float32)
    c = _codes(rng, T, H, P, N, G, dt_value=1.0, A_value=0.0, h0=h0, small=True)
    y_ref, h_ref, _ = oracle.ssd(c, threads=1)
    assert np.max(np.abs(h_ref)) < 2048                      # integers below 2^11: exact in binary16
    y16, h16, _ = oracle.ssd(c, threads=1, state_f16=True)
    assert np.array_equal(h16, h_ref) and np.array_equal(y16, y_ref)


def test_one_token_by_brute_force():
    """One step from a binary16 state: the update in double, then rounded to binary16 (numpy's
    conversion); y from the update before rounding."""
    rng = np.random.default_rng(7)
    H, P, N, G = 4, 8, 16, 2
    h0 = (rng.standard_normal((1, H, P, N)) * 3).astype(np.float16).astype(np.float32)
    c = _codes(rng, 1, H, P, N, G, h0=h0)
    y16, h16, _ = oracle.ssd(c, threads=1, state_f16=True)
    for h in range(H):
        g = h // (H // G)
        a = np.exp(np.float64(c.dt[0, 0, h]) * np.float64(c.A[h]))
        x = np.float64(c.sx[h]) * c.qx[0, 0, h].astype(np.float64)
        Bv = np.float64(c.sB[g]) * c.qB[0, 0, g].astype(np.float64)
        Cv = np.float64(c.sC[g]) * c.qC[0, 0, g].astype(np.float64)
        upd = a * h0[0, h].astype(np.float64) + np.float64(c.dt[0, 0, h]) * x[:, None] * Bv[None, :]
        y = upd @ Cv + np.float64(c.D[h]) * x
        assert np.allclose(y16[0, 0, h], y, rtol=1e-12, atol=1e-12)
        assert np.array_equal(h16[0, h], upd.astype(np.float16).astype(np.float64))


def test_error_stays_within_one_rounding_per_step():
    """|h_cached - h_exact| <= T half-ulps of the largest state: each step adds at most one
    rounding of 2^-11 relative, and the decay exp(dt A) <= 1 never amplifies older errors."""
    rng = np.random.default_rng(8)
    T, H, P, N, G = 64, 3, 8, 16, 1
    h0 = (rng.standard_normal((1, H, P, N)) * 0.5).astype(np.float16).astype(np.float32)
    c = _codes(rng, T, H, P, N, G, h0=h0)
    _, h_ref, traj = oracle.ssd(c, threads=1, chunk=1)        # traj: the state entering every token
    _, h16, _ = oracle.ssd(c, threads=1, state_f16=True)
    peak = max(np.nanmax(np.abs(traj)), np.max(np.abs(h_ref)))
    err = np.max(np.abs(h16 - h_ref))
    assert 0 < err <= T * 2.0 ** -11 * peak
