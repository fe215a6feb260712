"""Pins for the oracle's fp64 recurrence and chunk quantities (CPU only).

The recurrence is h_t = exp(dt_t A_h) h_{t-1} + dt_t B_t x_t, y_t = C_t . h_t + D_h x_t
(Ternary Mamba, Section 1, with the zero-order-hold decay), over dequantized
INT8 codes.  Each test below checks it against something that does not re-run
its loop: an independent chunked dual-form evaluation, closed forms, a
hand-worked example, and invariants of a linear time-varying system,
including the error-propagation formula of Ternary Mamba Section 6.2 (eq. 2).
"""
import math

import numpy as np
import pytest

import oracle
from ref_chunked import chunked_ssd, dequantize


def _codes(seed, b=2, L=37, H=4, P=3, N=5, G=2, h0=True, dt_scale=1.0):
    rng = np.random.default_rng(seed)
    qx = rng.integers(-127, 128, size=(b, L, H, P), dtype=np.int8)
    qB = rng.integers(-127, 128, size=(b, L, G, N), dtype=np.int8)
    qC = rng.integers(-127, 128, size=(b, L, G, N), dtype=np.int8)
    sx = rng.uniform(0.005, 0.05, size=H).astype(np.float32)
    sB = rng.uniform(0.005, 0.05, size=G).astype(np.float32)
    sC = rng.uniform(0.005, 0.05, size=G).astype(np.float32)
    dt = (np.log1p(np.exp(rng.normal(-2, 0.5, size=(b, L, H)))) * dt_scale).astype(np.float32)
    A = (-np.exp(rng.uniform(0, math.log(16), size=H))).astype(np.float32)
    D = rng.uniform(0.5, 1.5, size=H).astype(np.float32)
    h = rng.normal(0, 0.1, size=(b, H, P, N)).astype(np.float32) if h0 else None
    return oracle.Codes(qx, sx, qB, sB, qC, sC, dt, A, D, h)


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


@pytest.mark.parametrize("chunk", [1, 3, 16, 64, 37])
def test_matches_independent_chunked_form(chunk):
    c = _codes(1)
    y, hf, bounds = oracle.ssd(c, chunk=chunk, threads=1)
    ref = chunked_ssd(c.qx, c.sx, c.qB, c.sB, c.qC, c.sC, c.dt, c.A, c.D, c.h0, chunk=chunk)
    assert _rel(y, ref["y"]) < 1e-12
    assert _rel(hf, ref["h_final"]) < 1e-12
    assert _rel(bounds, ref["Hprev"]) < 1e-12


def test_chunked_form_ragged_and_whole_sequence_dual():
    # L = 250 with chunk 64 (ragged tail of 58) and chunk = L (the quadratic dual of the whole sequence)
    c = _codes(2, b=1, L=250, H=2, P=4, N=6, G=1)
    y, hf, _ = oracle.ssd(c, threads=1)
    for q in (64, 250):
        ref = chunked_ssd(c.qx, c.sx, c.qB, c.sB, c.qC, c.sC, c.dt, c.A, c.D, c.h0, chunk=q)
        assert _rel(y, ref["y"]) < 1e-11
        assert _rel(hf, ref["h_final"]) < 1e-11


def test_no_decay_is_a_prefix_sum():
    # A = 0: h_t = h0 + sum_{s<=t} dt_s x_s B_s^T, y_t = C_t . h_t + D x_t
    c = _codes(3)
    c.A[:] = 0
    y, hf, _ = oracle.ssd(c, threads=1)
    x, B, C = dequantize(c.qx, c.sx, c.qB, c.sB, c.qC, c.sC)
    u = c.dt.astype(np.float64)[..., None, None] * x[..., :, None] * B[..., None, :]   # (b,L,H,P,N)
    hs = np.cumsum(u, axis=1) + c.h0.astype(np.float64)[:, None]
    y_cf = np.einsum("blhn,blhpn->blhp", C, hs) + c.D.astype(np.float64)[None, None, :, None] * x
    assert _rel(y, y_cf) < 1e-12
    assert _rel(hf, hs[:, -1]) < 1e-12


def test_decay_to_zero_closed_form():
    # A = -1e5: exp(dt A) underflows to exactly 0, so h_t = dt_t x_t B_t^T and
    # y_t = (C_t . B_t) dt_t x_t + D x_t
    c = _codes(4)
    c.A[:] = -1e5
    y, hf, _ = oracle.ssd(c, threads=1)
    x, B, C = dequantize(c.qx, c.sx, c.qB, c.sB, c.qC, c.sC)
    dt = c.dt.astype(np.float64)
    cb = np.einsum("blhn,blhn->blh", C, B)
    y_cf = cb[..., None] * dt[..., None] * x + c.D.astype(np.float64)[None, None, :, None] * x
    assert _rel(y, y_cf) < 1e-13
    h_cf = dt[:, -1, :, None, None] * x[:, -1, :, :, None] * B[:, -1, :, None, :]
    assert _rel(hf, h_cf) < 1e-13


def test_zero_B_and_zero_C():
    c = _codes(5)
    x, _, _ = dequantize(c.qx, c.sx, c.qB, c.sB, c.qC, c.sC)
    c0 = _codes(5)
    c0.qB[:] = 0
    c0.h0 = None
    y, hf, _ = oracle.ssd(c0, threads=1)
    assert np.array_equal(y, c.D.astype(np.float64)[None, None, :, None] * x)   # exactly D x
    assert np.all(hf == 0)
    c1 = _codes(5)
    c1.qC[:] = 0
    y1, hf1, _ = oracle.ssd(c1, threads=1)
    assert np.array_equal(y1, c.D.astype(np.float64)[None, None, :, None] * x)
    assert np.max(np.abs(hf1)) > 0


def test_hand_worked_scalar_sequence():
    # H = P = N = G = 1, three tokens, worked by hand:
    #   x = 0.5 * [2, -1, 3] = [1, -0.5, 1.5];  B = [1, 2, -1];  C = 0.25 * [1, 1, 2]
    #   dt = [0.5, 0.25, 1], A = -2 -> decays exp(-1), exp(-0.5), exp(-2);  D = 1;  h0 = 0.5
    #   h_0 = 0.5 e^-1 + 0.5 * 1 * 1          y_0 = 0.25 h_0 + 1
    #   h_1 = e^-0.5 h_0 + 0.25 * (-0.5) * 2   y_1 = 0.25 h_1 - 0.5
    #   h_2 = e^-2 h_1 + 1 * 1.5 * (-1)        y_2 = 0.5 h_2 + 1.5
    c = oracle.Codes(np.array([2, -1, 3], np.int8).reshape(1, 3, 1, 1), np.array([0.5], np.float32),
                     np.array([1, 2, -1], np.int8).reshape(1, 3, 1, 1), np.array([1.0], np.float32),
                     np.array([1, 1, 2], np.int8).reshape(1, 3, 1, 1), np.array([0.25], np.float32),
                     np.array([0.5, 0.25, 1.0], np.float32).reshape(1, 3, 1), np.array([-2.0], np.float32),
                     np.array([1.0], np.float32), np.array([0.5], np.float32).reshape(1, 1, 1, 1))
    y, hf, _ = oracle.ssd(c, threads=1)
    h0 = 0.5 * math.exp(-1) + 0.5
    h1 = math.exp(-0.5) * h0 - 0.25
    h2 = math.exp(-2) * h1 - 1.5
    expect = [0.25 * h0 + 1, 0.25 * h1 - 0.5, 0.5 * h2 + 1.5]
    assert np.allclose(y.reshape(-1), expect, rtol=0, atol=1e-15)
    assert abs(hf.reshape(-1)[0] - h2) < 1e-15


def test_single_token():
    # L = 1: h = exp(dt A) h0 + dt x B^T; y = C . h + D x
    c = _codes(6, L=1)
    y, hf, _ = oracle.ssd(c, threads=1)
    x, B, C = dequantize(c.qx, c.sx, c.qB, c.sB, c.qC, c.sC)
    dt = c.dt.astype(np.float64)[:, 0]
    a = np.exp(dt * c.A.astype(np.float64))
    h = a[..., None, None] * c.h0 + dt[..., None, None] * x[:, 0, :, :, None] * B[:, 0, :, None, :]
    assert _rel(hf, h) < 1e-14
    y_cf = np.einsum("bhn,bhpn->bhp", C[:, 0], h) + c.D[None, :, None] * x[:, 0]
    assert _rel(y[:, 0], y_cf) < 1e-14


def test_group_mapping_contiguous_blocks():
    # H = 4, G = 2: heads 0,1 read group 0 and heads 2,3 read group 1.
    c = _codes(7, H=4, G=2, h0=False)
    c.qB[:, :, 1, :] = 0
    y, hf, _ = oracle.ssd(c, threads=1)
    assert np.max(np.abs(hf[:, :2])) > 0
    assert np.all(hf[:, 2:] == 0)


def test_superposition_and_head_homogeneity():
    c = _codes(8)
    y, hf, _ = oracle.ssd(c, threads=1)
    c_x = _codes(8)
    c_x.h0 = None
    y_x, hf_x, _ = oracle.ssd(c_x, threads=1)
    c_h = _codes(8)
    c_h.qx[:] = 0
    y_h, hf_h, _ = oracle.ssd(c_h, threads=1)
    assert _rel(y, y_x + y_h) < 1e-12
    assert _rel(hf, hf_x + hf_h) < 1e-12
    # doubling one head's x scale doubles exactly that head's input-driven response
    c2 = _codes(8)
    c2.h0 = None
    c2.sx[1] *= 2
    y2, hf2, _ = oracle.ssd(c2, threads=1)
    assert np.array_equal(y2[:, :, 1], 2 * y_x[:, :, 1])
    assert np.array_equal(hf2[:, 1], 2 * hf_x[:, 1])
    others = [0, 2, 3]
    assert np.array_equal(y2[:, :, others], y_x[:, :, others])


def test_split_invariance():
    # run(L) == run(L - L1, h0 = h_final(run(L1)))
    c = _codes(9, L=50)
    y, hf, _ = oracle.ssd(c, threads=1)
    L1 = 21
    a = oracle.Codes(c.qx[:, :L1], c.sx, c.qB[:, :L1], c.sB, c.qC[:, :L1], c.sC, c.dt[:, :L1], c.A, c.D, c.h0)
    ya, hfa, _ = oracle.ssd(a, threads=1)
    # the carried state is fp64 here, so pass it through a float64-capable path: rerun tail
    # with h0 rounded to fp32 and compare with the tolerance that rounding implies
    b = oracle.Codes(c.qx[:, L1:], c.sx, c.qB[:, L1:], c.sB, c.qC[:, L1:], c.sC, c.dt[:, L1:], c.A, c.D,
                     hfa.astype(np.float32))
    yb, hfb, _ = oracle.ssd(b, threads=1)
    assert _rel(ya, y[:, :L1]) < 1e-14
    assert _rel(yb, y[:, L1:]) < 1e-6
    assert _rel(hfb, hf) < 1e-6


def test_error_propagation_eq2():
    # A perturbation e of x at token t0 changes the state at T by Abar^(T - t0) applied to
    # dt x-perturbation B^T (Ternary Mamba, Section 6.2, eq. 2, with a constant decay Abar
    # obtained from a constant dt).
    c = _codes(10, b=1, L=40, H=1, P=2, N=3, G=1, h0=False)
    c.dt[:] = np.float32(0.125)
    y, hf, _ = oracle.ssd(c, threads=1)
    t0 = 13
    c2 = _codes(10, b=1, L=40, H=1, P=2, N=3, G=1, h0=False)
    c2.dt[:] = np.float32(0.125)
    c2.qx[0, t0, 0, 1] = np.int8(int(c2.qx[0, t0, 0, 1]) + (5 if c2.qx[0, t0, 0, 1] < 100 else -5))
    y2, hf2, _ = oracle.ssd(c2, threads=1)
    dq = float(int(c2.qx[0, t0, 0, 1]) - int(c.qx[0, t0, 0, 1]))
    abar = math.exp(0.125 * float(c.A[0]))
    eps = 0.125 * dq * float(c.sx[0]) * c.qB[0, t0, 0].astype(np.float64) * float(c.sB[0])
    T = 39
    dh = hf2[0, 0] - hf[0, 0]
    expect = np.zeros_like(dh)
    expect[1] = abar ** (T - t0) * eps
    assert np.max(np.abs(dh - expect)) < 1e-12 * max(1.0, np.max(np.abs(hf)))
    # the output is untouched before t0
    assert np.array_equal(y2[0, :t0], y[0, :t0])


def test_chunk_cumsum_constant_dt():
    c = _codes(11, b=1, L=70, H=2, G=1, h0=False)
    c.dt[:] = np.float32(0.25)
    acs = oracle.chunk_cumsum(c, 0, 1, 32)
    for cidx in range(3):
        n = min(32, 70 - 32 * cidx)
        expect = 0.25 * float(c.A[1]) * np.arange(1, n + 1)
        assert np.allclose(acs[cidx, :n], expect, rtol=0, atol=1e-12)


@pytest.mark.parametrize("chunk", [8, 16, 37])
def test_chunk_state_links_boundary_states(chunk):
    # H_{c+1} = exp(Acs[c, last]) H_c + S_c, with H_c taken from the sequential recurrence
    c = _codes(12, b=1, L=37, H=2, G=1)
    _, hf, bounds = oracle.ssd(c, chunk=chunk, threads=1)
    for h in range(c.H):
        S = oracle.chunk_state(c, 0, h, chunk)
        acs = oracle.chunk_cumsum(c, 0, h, chunk)
        nc = S.shape[0]
        for ci in range(nc):
            n = min(chunk, c.L - ci * chunk)
            nxt = hf[0, h] if ci == nc - 1 else bounds[0, ci + 1, h]
            pred = math.exp(acs[ci, n - 1]) * bounds[0, ci, h] + S[ci]
            assert _rel(pred, nxt) < 1e-12


def test_threads_do_not_change_results():
    c = _codes(13, b=3, H=4)
    y1, h1, _ = oracle.ssd(c, threads=1)
    y4, h4, _ = oracle.ssd(c, threads=4)
    assert np.array_equal(y1, y4) and np.array_equal(h1, h4)


def test_sampled_pairs_only_fill_those_pairs():
    c = _codes(14, b=2, H=4)
    y, hf, _ = oracle.ssd(c, pairs=[(1, 2)], threads=1)
    assert np.all(np.isfinite(y[1, :, 2])) and np.all(np.isnan(y[0]))
