"""GPU parity of ssdq_state_update_i8: the decode step with the state cached as 8-bit codes and
one binary32 scale per state row.

One step from the same cached state.  The oracle forms the update u in double, the kernel in
fp32, so their row maxima m and scales s = binary32(m / 127) may differ by the fp32 rounding of
the update, and a code may differ only where u / s lies within the kernel's rounding of a
midpoint between two codes (there either neighbour is a correct rounding).  The band is derived
per element from the kernel's arithmetic (unit roundoff e = 2^-24):
  - e^(dt A) by exp2 of a rounded product: relative error <= (1.5 |dt A| + 1) 2e;
  - u = fma(e^(dt A) s_old, q_old, ((dt s_x) s_B) x) b): with T1 = e^(dt A) s_old q_old and
    T2 = dt xhat Bhat, |u_gpu - u| <= |T1| (eps_exp + 2e) + |T2| 4e + |u| e  =: du;
  - |m_gpu - m| <= max_n du =: dm, and the kernel's scale is within one ulp of binary32(m_gpu / 127)
    (its division sequence is checked over every binary32 significand on the host), so
    |s_gpu - s| <= dm / 127 + 2 ulp(s);
  - the kernel's quotient u_gpu rcp(s_gpu) (reciprocal within an ulp) is rounded to the nearest
    integer exactly, so |t_gpu - u / s| <= du / s + |u / s| (|s_gpu - s| / s + 2e), with |u / s| <= 127.5.
Twice that bound is the band: about 2^-14 code units for a slowly decaying row, up to about
2^-11 for rows whose decay |dt A| is near 5 (the exp's error grows with its argument).  Over many
steps each such flip moves one element by a code step and then decays, and once a row's largest
elements differ its scale differs too, so the two caches drift apart by a few code steps of a
slowly decaying row; the multi-step tests bound that drift per row from the oracle's own scales
(see _caching_bound) and hold y to the usual tolerance.  Starting codes and scales come from the
oracle's own re-quantization of the seeded fp32 state."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import Y_TOL, dev, note, threaded, to_dev

pytestmark = pytest.mark.gpu

EPS = 2.0 ** -24       # binary32 unit roundoff
ULP = 2.0 ** -23       # binary32 ulp relative to a normal value (upper bound)
SAFETY = 2.0


def _one_step_bounds(c, b, h, q0, s0, u, s_ref):
    """Per-row bound on |s_gpu - s_ref| and per-element band on the quotient u / s (code units)
    of one step from the cached codes q0, scales s0 (see the module docstring)."""
    g = h // (c.H // c.G)
    dt = float(c.dt[b, 0, h])
    dA = abs(dt * float(c.A[h]))
    eps_exp = (1.5 * dA + 1.0) * 2 * EPS
    T1 = np.exp(dt * float(c.A[h])) * s0[b, h].astype(np.float64)[:, None] * q0[b, h]
    xhat = float(c.sx[h]) * c.qx[b, 0, h].astype(np.float64)
    bhat = float(c.sB[g]) * c.qB[b, 0, g].astype(np.float64)
    T2 = dt * xhat[:, None] * bhat[None, :]
    du = np.abs(T1) * (eps_exp + 2 * EPS) + np.abs(T2) * 4 * EPS + np.abs(u) * EPS
    dm = du.max(axis=1)
    s = s_ref.astype(np.float64)
    ds = dm / 127 + 2 * ULP * s
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(s[:, None] > 0, u / s[:, None], 0.0)
        band = np.where(s[:, None] > 0, du / s[:, None] + np.abs(t) * (ds / s + 2 * EPS)[:, None], 0.0)
    return SAFETY * ds, SAFETY * band, t


def _start(dec):
    """The seeded fp32 starting state as 8-bit codes and row scales (the oracle's re-quantization)."""
    st = dec["state"]
    b, H, P, N = st.shape
    q, s, _ = oracle.requantize_rows_i8(st.reshape(-1, N).astype(np.float64))
    return q.reshape(b, H, P, N), s.reshape(b, H, P)


def _gpu_decode_i8(dec, q0, s0, with_D=True):
    """Quantize every step's x, B, C and run the steps on the 8-bit state; returns
    (y (T,b,H,P), final codes, final scales)."""
    import quantized_selective_state_amd as ssdq
    sx, sB, sC = to_dev(dec["x_scale"]), to_dev(dec["B_scale"]), to_dev(dec["C_scale"])
    qx = ssdq.quantize(to_dev(dec["x16"]), sx)
    qB = ssdq.quantize(to_dev(dec["B16"]), sB)
    qC = ssdq.quantize(to_dev(dec["C16"]), sC)
    dt, A = to_dev(dec["dt"]), to_dev(dec["A"])
    D = to_dev(dec["D"]) if with_D else None
    state, scale = to_dev(q0), to_dev(s0)
    T = dec["x16"].shape[0]
    ys = torch.empty((T,) + tuple(qx.shape[1:]), dtype=torch.float16, device=dev())
    for t in range(T):
        ssdq.state_update(state, qx[t], sx, qB[t], sB, qC[t], sC, dt[t], A, D, y=ys[t], state_scale=scale)
    torch.cuda.synchronize()
    return ys.float().cpu().numpy(), state.cpu().numpy(), scale.cpu().numpy()


def _small(seed, b, H, P, N, G, T):
    shape = workloads.DecodeShape(f"dec8_{seed}", b, T, H, P, N, G, 0.5)
    return workloads.make_decode(shape, seed_index=seed)


def _caching_bound(c, b, h, s0, steps):
    """Per-row bound on |g_T - o_T| after T steps, g the GPU's cached state and o the oracle's,
    both starting from the same codes.  With e_t = max_n |g_t - o_t| of a row and a_t = e^(dt_t A):
    each step the two updates differ by at most a_t e_t plus the kernel's fp32 error err_t, each
    side re-quantizes within half its own scale, and the GPU's scale exceeds the oracle's s_{t+1}
    by at most max|u_g - u_o| / 127, so e_{t+1} <= (a_t e_t + err_t)(1 + 1/254) + s_{t+1}, with
    err_t <= 127 (a_t s_t + s_{t+1})(eps_exp + 6e) (the one-step analysis of the module docstring).
    A rounding flip near a midpoint moves an element by one code step and then decays with a_t, so
    over many steps of a slowly decaying head the two caches drift apart by several code steps
    (each bounded, none accumulating without decay)."""
    dts = c.dt[b, :, h].astype(np.float64)
    A = float(c.A[h])
    s_prev = s0[b, h].astype(np.float64)
    e = np.zeros_like(s_prev)
    for t in range(c.L):
        a = np.exp(dts[t] * A)
        eps_exp = (1.5 * abs(dts[t] * A) + 1.0) * 2 * EPS
        s_new = steps[t].astype(np.float64)
        err = 127 * (a * s_prev + s_new) * (eps_exp + 6 * EPS)
        e = (a * e + err) * (1 + 1 / 254) + s_new
        s_prev = s_new
    return e * (1 + 1e-6)


def _check_steps(dec, q0, s0, y, q, s, tag=""):
    """Every (b, h) sequence against the oracle with the same caching (run on host threads, each
    sequence reduced to its maxima at once): the decoded cached states within the derived drift
    bound of every row, and y within the bar."""
    c = oracle.decode_as_prefill(dec)

    def one(bh):
        b, h = bh
        y8, h8, _, s8, _, steps = oracle.ssd_one_state_i8(c, b, h, q0, s0, scales_per_step=True)
        got = s[b, h].astype(np.float64)[:, None] * q[b, h]
        err = np.abs(got - h8).max(axis=1)                                  # per row
        bound = _caching_bound(c, b, h, s0, steps)
        row_step = np.maximum(s8.astype(np.float64), s[b, h])             # one code step of each row
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
            in_steps = np.where(row_step > 0, err / row_step, 0.0)
        return (bool(np.all(err <= bound)), float(ratio.max()), float(in_steps.max()), float(np.max(np.abs(y8))),
                float(np.max(np.abs(y[:, b, h] - y8))))

    r = threaded(one, [(b, h) for b in range(c.batch) for h in range(c.H)])
    worst_ratio = max(v[1] for v in r)
    steps = np.array([v[2] for v in r])
    ymax = max(v[3] for v in r)
    e_y = max(v[4] for v in r)
    note(f"{tag} ({len(r)} sequences): cached states within {worst_ratio:.2f} of the derived drift bound; "
         f"worst row {steps.max():.2f} code steps from the cached oracle (99th percentile of sequences "
         f"{np.percentile(steps, 99):.2f}); y {e_y / ymax:.2e}")
    assert all(v[0] for v in r), "a cached state drifted beyond its derived bound"
    assert e_y <= Y_TOL * ymax


def test_one_step_codes_match_the_oracle():
    dec = _small(70, b=4, H=8, P=64, N=128, G=2, T=1)
    q0, s0 = _start(dec)
    y, q, s = _gpu_decode_i8(dec, q0, s0)
    c = oracle.decode_as_prefill(dec)
    near = mism = total = s_exact = s_rows = 0
    worst_band = 0.0
    for b in range(c.batch):
        for h in range(c.H):
            y8, _, q8, s8, u = oracle.ssd_one_state_i8(c, b, h, q0, s0)
            ds, band, t = _one_step_bounds(c, b, h, q0, s0, u, s8)
            assert np.all(np.abs(s[b, h].astype(np.float64) - s8) <= ds), "row scale beyond its derived bound"
            s_exact += int(np.sum(s[b, h] == s8))
            s_rows += s8.size
            near_mid = np.abs(np.abs(t - np.floor(t)) - 0.5) <= band
            diff = q[b, h].astype(np.int32) - q8
            assert np.all(diff[~near_mid] == 0), "a code differs away from a rounding midpoint"
            qb = q[b, h][near_mid].astype(np.float64)
            tb = np.clip(t[near_mid], -127, 127)
            assert np.all((qb == np.floor(tb)) | (qb == np.ceil(tb)))   # either neighbour of the quotient
            near += int(near_mid.sum())
            mism += int(np.count_nonzero(diff))
            total += diff.size
            worst_band = max(worst_band, float(band.max()))
            assert np.max(np.abs(y[0, b, h] - y8[0])) <= Y_TOL * max(np.max(np.abs(y8)), 1e-30)
    note(f"one step: {total} codes, {near} within the derived midpoint band (widest {worst_band:.2e} code "
         f"units), {mism} differ; {s_exact} of {s_rows} row scales equal the oracle's")
    # the widest bands belong to strongly decaying rows (|dt A| near 5), where the fp32 exp of the
    # decay contributes most: still below 2^-10 of a code step
    assert worst_band < 2.0 ** -10
    assert near < total // 1000


@pytest.mark.parametrize("N,G", [(128, 4), (64, 2)])
def test_small_decode_every_step(N, G):
    dec = _small(71 + N, b=4, H=8, P=64, N=N, G=G, T=16)
    q0, s0 = _start(dec)
    y, q, s = _gpu_decode_i8(dec, q0, s0)
    _check_steps(dec, q0, s0, y, q, s, tag=f"i8 state N={N}")


def test_headdim_below_64_and_no_D():
    dec = _small(74, b=3, H=4, P=48, N=128, G=2, T=8)
    dec["D"] = None
    q0, s0 = _start(dec)
    y, q, s = _gpu_decode_i8(dec, q0, s0, with_D=False)
    _check_steps(dec, q0, s0, y, q, s, tag="i8 state P=48 no D")


def test_zero_and_subnormal_scale_rows_are_flushed():
    """Rows without input stay zero when they start at zero (no 0/0), and rows so small that
    their scale would be subnormal (here a starting scale of 1e-39) are flushed to zero codes
    and scale 0, as the oracle does."""
    dec = _small(75, b=2, H=4, P=64, N=128, G=1, T=2)
    dec["x16"][:, :, :, :16] = 0           # rows p < 16 of every head get no input
    q0, s0 = _start(dec)
    q0[:, :, :8] = 0
    s0[:, :, :8] = 0
    s0[:, :, 8:16] = np.float32(1e-39)
    y, q, s = _gpu_decode_i8(dec, q0, s0)
    assert not np.any(q[:, :, :16]) and not np.any(s[:, :, :16])
    _check_steps(dec, q0, s0, y, q, s, tag="i8 state zero rows")


def test_full_decode_workload():
    """batch 256, 128 heads, 8 groups, 128 steps on the 256 MiB 8-bit state: every (batch, head)
    sequence against the oracle with the same caching."""
    note("generating decode workload")
    dec = workloads.make_decode("mamba2-8b-decode")
    q0, s0 = _start(dec)
    note("gpu decode 128 steps, 8-bit state")
    y, q, s = _gpu_decode_i8(dec, q0, s0)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(s))
    note("oracle decode, 8-bit state: all sequences")
    _check_steps(dec, q0, s0, y, q, s, tag="i8 state full")
