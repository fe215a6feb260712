"""Pins for the oracle's 8-bit cached state (the decode state kept between tokens as 8-bit codes
with one binary32 scale per state row, the 8-bit cached states of the Quamba2 rebuttal's
Tables R7/R8).

The re-quantization is checked against exact rational arithmetic (the scale is the binary32
value nearest to max|row| / 127, each code the exact quotient rounded half to even), on
hand-made ties and on the special rows; the recurrence where the pages' arithmetic fixes the
answer (states that are small integers with a row maximum of 127: no rounding at all), by
brute force on one token, under an exact power-of-two rescaling, and against the error bound
that one re-quantization per token implies."""
from fractions import Fraction

import numpy as np

import oracle


def _f32_nearest(v: Fraction) -> float:
    """The binary32 value nearest to the rational v (ties to even), by search over the two
    binary32 neighbours of the double nearest to v."""
    d = np.float32(float(v))
    cands = {float(d), float(np.nextafter(d, np.float32(np.inf))), float(np.nextafter(d, np.float32(-np.inf)))}
    best = sorted(cands, key=lambda c: (abs(Fraction(c) - v), int(np.float32(c).view(np.uint32)) & 1))
    return best[0]


def test_requantize_matches_exact_rationals():
    rng = np.random.default_rng(11)
    rows = rng.standard_normal((40, 32)) * 10.0 ** rng.integers(-6, 6, (40, 1))
    q, s, dec = oracle.requantize_rows_i8(rows)
    for r in range(rows.shape[0]):
        m = max(abs(Fraction(v)) for v in rows[r])
        assert s[r] == _f32_nearest(m / 127)
        for n in range(rows.shape[1]):
            t = Fraction(rows[r, n]) / Fraction(float(s[r]))
            want = max(-127, min(127, round(t)))          # Fraction rounds half to even
            assert q[r, n] == want
            assert dec[r, n] == float(s[r]) * want
        assert np.max(np.abs(q[r])) == 127                # the largest magnitude takes the end code
        assert np.all(np.abs(dec[r] - rows[r]) <= float(s[r]) / 2 * (1 + 1e-12))


def test_ties_go_to_even_codes_and_special_rows():
    row = np.array([127.0, 0.5, 1.5, 2.5, -0.5, -2.5, 3.5, -126.5, 0.0, 64.0])
    q, s, dec = oracle.requantize_rows_i8(row)
    assert s[0] == 1.0
    assert list(q[0]) == [127, 0, 2, 2, 0, -2, 4, -126, 0, 64]
    assert np.array_equal(dec[0], q[0].astype(np.float64))
    # a negative largest element, and a zero row
    q, s, dec = oracle.requantize_rows_i8(np.array([[-254.0, 1.0, 3.0, 127.0], [0.0, 0.0, 0.0, 0.0]]))
    assert s[0] == 2.0 and list(q[0]) == [-127, 0, 2, 64]   # 1/2 -> 0, 3/2 -> 2, 127/2 -> 64
    assert s[1] == 0.0 and not np.any(q[1]) and not np.any(dec[1])
    # a row whose scale would be subnormal is flushed; one just above keeps its codes
    q, s, dec = oracle.requantize_rows_i8(np.array([[1e-37, -5e-38, 0.0], [127 * 2.0 ** -126, 2.0 ** -126, 0.0]]))
    assert s[0] == 0.0 and not np.any(q[0]) and not np.any(dec[0])
    assert s[1] == np.float32(2.0 ** -126) and list(q[1]) == [127, 1, 0]


def _codes(rng, T, H, P, N, G, small=False):
    lo, hi = (-3, 4) if small else (-127, 128)
    qx = rng.integers(lo, hi, (1, T, H, P)).astype(np.int8)
    qB = rng.integers(lo, hi, (1, T, G, N)).astype(np.int8)
    qC = rng.integers(-127, 128, (1, T, G, N)).astype(np.int8)
    one = lambda n: np.ones(n, np.float32)
    if small:
        sx, sB, sC = one(H), one(G), one(G)
        dt = np.ones((1, T, H), np.float32)
        A = np.zeros(H, np.float32)
    else:
        sx = rng.uniform(0.01, 0.05, H).astype(np.float32)
        sB = rng.uniform(0.01, 0.05, G).astype(np.float32)
        sC = rng.uniform(0.01, 0.05, G).astype(np.float32)
        dt = rng.uniform(0.001, 0.1, (1, T, H)).astype(np.float32)
        A = -rng.uniform(1, 16, H).astype(np.float32)
    D = rng.uniform(0.5, 1.5, H).astype(np.float32)
    return qx, sx, qB, sB, qC, sC, dt, A, D


def test_integer_states_with_row_max_127_are_not_rounded():
    """No decay (A = 0), dt = 1, unit scales, column 0 of every row held at 127 (B[:, 0] = 0)
    and the other entries kept small: every state is an integer row with maximum 127, so the
    scale is 1, the codes are the state itself, and caching changes nothing."""
    rng = np.random.default_rng(12)
    T, H, P, N, G = 10, 2, 4, 8, 1
    qx, sx, qB, sB, qC, sC, dt, A, D = _codes(rng, T, H, P, N, G, small=True)
    qB[..., 0] = 0
    q0 = rng.integers(-30, 31, (1, H, P, N)).astype(np.int8)
    q0[..., 0] = 127
    s0 = np.ones((1, H, P), np.float32)
    exact = oracle.Codes(qx, sx, qB, sB, qC, sC, dt, A, D, q0.astype(np.float32))
    cached = oracle.Codes(qx, sx, qB, sB, qC, sC, dt, A, D)
    for h in range(H):
        y_ref, h_ref, _ = oracle.ssd_one(exact, 0, h)
        y8, h8, q, s, _ = oracle.ssd_one_state_i8(cached, 0, h, q0, s0)
        assert np.max(np.abs(h_ref)) == 127
        assert np.array_equal(h8, h_ref) and np.array_equal(y8, y_ref)
        assert np.array_equal(q.astype(np.float64), h_ref) and np.all(s == 1.0)


def test_one_token_by_brute_force():
    """One step from 8-bit codes: decode, update in double, y from the update, then each row
    re-quantized (checked here with exact rationals)."""
    rng = np.random.default_rng(13)
    H, P, N, G = 4, 6, 16, 2
    qx, sx, qB, sB, qC, sC, dt, A, D = _codes(rng, 1, H, P, N, G)
    q0 = rng.integers(-127, 128, (1, H, P, N)).astype(np.int8)
    s0 = rng.uniform(0.01, 0.1, (1, H, P)).astype(np.float32)
    c = oracle.Codes(qx, sx, qB, sB, qC, sC, dt, A, D)
    for h in range(H):
        g = h // (H // G)
        a = np.exp(np.float64(dt[0, 0, h]) * np.float64(A[h]))
        x = np.float64(sx[h]) * qx[0, 0, h].astype(np.float64)
        Bv = np.float64(sB[g]) * qB[0, 0, g].astype(np.float64)
        Cv = np.float64(sC[g]) * qC[0, 0, g].astype(np.float64)
        h0 = s0[0, h].astype(np.float64)[:, None] * q0[0, h].astype(np.float64)
        upd = a * h0 + np.float64(dt[0, 0, h]) * x[:, None] * Bv[None, :]
        y, h8, q, s, u = oracle.ssd_one_state_i8(c, 0, h, q0, s0)
        assert np.allclose(u, upd, rtol=1e-13, atol=0)
        assert np.allclose(y[0], upd @ Cv + np.float64(D[h]) * x, rtol=1e-12, atol=1e-12)
        for p in range(P):
            m = max(abs(Fraction(v)) for v in u[p])
            assert s[p] == _f32_nearest(m / 127)
            want = [max(-127, min(127, round(Fraction(v) / Fraction(float(s[p]))))) for v in u[p]]
            assert list(q[p]) == want
            assert np.array_equal(h8[p], float(s[p]) * np.array(want, np.float64))


def test_power_of_two_rescaling_is_exact():
    """Scaling x's scale and the starting state's scales by 4 scales every update, hence every
    row maximum and scale, by exactly 4: the codes are unchanged and y and the state scale by 4."""
    rng = np.random.default_rng(14)
    T, H, P, N, G = 12, 2, 4, 16, 1
    qx, sx, qB, sB, qC, sC, dt, A, D = _codes(rng, T, H, P, N, G)
    q0 = rng.integers(-127, 128, (1, H, P, N)).astype(np.int8)
    s0 = rng.uniform(0.01, 0.1, (1, H, P)).astype(np.float32)
    c1 = oracle.Codes(qx, sx, qB, sB, qC, sC, dt, A, D)
    c4 = oracle.Codes(qx, sx * 4, qB, sB, qC, sC, dt, A, D)
    for h in range(H):
        y1, h1, q1, s1, _ = oracle.ssd_one_state_i8(c1, 0, h, q0, s0)
        y4, h4, q4, s4, _ = oracle.ssd_one_state_i8(c4, 0, h, q0, s0 * 4)
        assert np.array_equal(q1, q4) and np.array_equal(s4, s1 * 4)
        assert np.array_equal(h4, h1 * 4) and np.array_equal(y4, y1 * 4)


def test_error_stays_within_one_requantization_per_step():
    """|h_cached - h_exact| <= sum over tokens of half a code step: each token's re-quantization
    moves an element by at most s / 2 = max|row| / 254 (plus the binary32 rounding of s), and the
    decay exp(dt A) <= 1 never amplifies older errors."""
    rng = np.random.default_rng(15)
    T, H, P, N, G = 48, 2, 6, 16, 1
    qx, sx, qB, sB, qC, sC, dt, A, D = _codes(rng, T, H, P, N, G)
    q0 = rng.integers(-127, 128, (1, H, P, N)).astype(np.int8)
    s0 = (rng.integers(40, 400, (1, H, P)) * 2.0 ** -12).astype(np.float32)   # 9-bit scales: s q exact in fp32
    h0 = (s0.astype(np.float64)[..., None] * q0).astype(np.float32)
    assert np.array_equal(h0.astype(np.float64), s0.astype(np.float64)[..., None] * q0)   # exact in fp32
    exact = oracle.Codes(qx, sx, qB, sB, qC, sC, dt, A, D, h0)
    cached = oracle.Codes(qx, sx, qB, sB, qC, sC, dt, A, D)
    for h in range(H):
        _, h_ref, traj = oracle.ssd_one(exact, 0, h, chunk=1)          # the state entering each token
        _, h8, _, _, _ = oracle.ssd_one_state_i8(cached, 0, h, q0, s0)
        peak = np.maximum(np.max(np.abs(traj), axis=(0, 2)), np.max(np.abs(h_ref), axis=1))   # per row
        err = np.max(np.abs(h8 - h_ref), axis=1)
        # the cached state's rows may exceed the exact ones by the accumulated error itself
        bound = T * (peak + err) / 254 * (1 + 1e-6)
        assert np.all(err > 0) and np.all(err <= bound)
