"""GPU parity of ssdq_state_update_i8: the decode step with the state cached as 8-bit codes and
one binary32 scale per state row.

One step from the same cached state: every code the oracle fixes is reproduced exactly.  The
oracle forms the update in double, the kernel in fp32; they can only part where the exact
quotient update / scale lies within fp32 rounding of a midpoint between two codes, and there
either neighbour is a correct rounding (checked), so the test compares the codes away from
midpoints and accepts either neighbour near one.  Over many steps such a flip moves one element
by one code step and decays afterwards, so the decoded states agree to a few code steps of their
row and y to the usual tolerance.  Starting codes and scales come from the oracle's own
re-quantization of the seeded fp32 state."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import Y_TOL, dev, note, sample_pairs, to_dev

pytestmark = pytest.mark.gpu

MIDPOINT_BAND = 2e-3   # |frac(u / s) - 1/2| below this: either neighbouring code is correct
FLIPS = 4              # code steps allowed over many steps for such flips


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


def _check_steps(dec, q0, s0, y, q, s, pairs=None, tag=""):
    c = oracle.decode_as_prefill(dec)
    if pairs is None:
        pairs = [(b, h) for b in range(c.batch) for h in range(c.H)]
    e_h = e_y = 0.0
    ymax = 0.0
    worst_steps = 0.0
    for b, h in pairs:
        y8, h8, _, s8, _ = oracle.ssd_one_state_i8(c, b, h, q0, s0)
        got = s[b, h].astype(np.float64)[:, None] * q[b, h]
        row_step = np.maximum(s8.astype(np.float64), s[b, h])[:, None]     # one code step of each row
        err = np.abs(got - h8)
        worst_steps = max(worst_steps, float(np.max(err / np.where(row_step > 0, row_step, 1.0))))
        assert np.all(err <= FLIPS * row_step * (1 + 1e-5) + 1e-30)
        ymax = max(ymax, np.max(np.abs(y8)))
        e_y = max(e_y, np.max(np.abs(y[:, b, h] - y8)))
        e_h = max(e_h, np.max(err))
    note(f"{tag}: state within {worst_steps:.2f} code steps of the cached oracle, y {e_y / ymax:.2e}")
    assert e_y <= Y_TOL * ymax


def test_one_step_codes_match_the_oracle():
    dec = _small(70, b=4, H=8, P=64, N=128, G=2, T=1)
    q0, s0 = _start(dec)
    y, q, s = _gpu_decode_i8(dec, q0, s0)
    c = oracle.decode_as_prefill(dec)
    near = mism = total = 0
    for b in range(c.batch):
        for h in range(c.H):
            y8, _, q8, s8, u = oracle.ssd_one_state_i8(c, b, h, q0, s0)
            assert np.allclose(s[b, h], s8, rtol=1e-5, atol=0)
            t = u / np.where(s8 > 0, s8.astype(np.float64), 1.0)[:, None]
            band = np.abs(np.abs(t - np.floor(t)) - 0.5) < MIDPOINT_BAND
            diff = q[b, h].astype(np.int32) - q8
            assert np.all(diff[~band] == 0)
            qb = q[b, h][band].astype(np.float64)
            tb = np.clip(t[band], -127, 127)
            assert np.all((qb == np.floor(tb)) | (qb == np.ceil(tb)))   # either neighbour of the quotient
            near += int(band.sum())
            mism += int(np.count_nonzero(diff))
            total += diff.size
            assert np.max(np.abs(y[0, b, h] - y8[0])) <= Y_TOL * max(np.max(np.abs(y8)), 1e-30)
    note(f"one step: {total} codes, {near} within the midpoint band, {mism} differ")
    assert near < total // 100


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


def test_full_decode_workload_sampled():
    """batch 256, 128 heads, 8 groups, 128 steps on the 256 MiB 8-bit state; oracle on sampled
    sequences (always with the largest and smallest x scales)."""
    note("generating decode workload")
    dec = workloads.make_decode("mamba2-8b-decode")
    q0, s0 = _start(dec)
    note("gpu decode 128 steps, 8-bit state")
    y, q, s = _gpu_decode_i8(dec, q0, s0)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(s))
    order = np.argsort(dec["x_scale"])
    pairs = sample_pairs(256, 128, 12, 23, list(order[-3:]) + list(order[:2]))
    note(f"oracle decode on {len(pairs)} sequences")
    _check_steps(dec, q0, s0, y, q, s, pairs=pairs, tag="i8 state full")
