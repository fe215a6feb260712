"""GPU parity of the output correction (SSDi8's per-channel mean correction): the corrected
prefill scan and the corrected decode step for the three state formats, against the oracle with
the same correction.

The correction is calibrated by the oracle on a separate calibration draw (the mean, per output
channel, of the unquantized scan's y minus the quantized scan's y).  The draws are one-sided
(x = m_h (N(0, 1) + 0.5)) and the x scales clip at the 90th percentile of |x|, so the quantized
inputs are biased and the correction is visibly nonzero; the test draw also checks that the
corrected output's mean error per channel is smaller than the uncorrected one's.  The pages print
no value of the correction, so this parity is pinned by the oracle's own identities only
(tests/test_oracle_correction.py)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import H_TOL, Y_TOL, gpu_quantize_inputs, note, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _pair(seed, batch=2, seqlen=320, nheads=8, headdim=64, dstate=128, ngroups=2, chunk=128, h0_std=0.1):
    shape = workloads.PrefillShape(f"corr{seed}", batch, seqlen, nheads, headdim, dstate, ngroups, chunk,
                                   "outlier_heads", "fixed_bias", h0_std)
    cal, test = workloads.make_calibrated_pair(shape, seed, x_mean=0.5, x_clip_pct=90.0)
    mu = oracle.mean_correction(cal)
    test["y_corr"] = mu
    return test, mu


def test_prefill_corrected_against_the_oracle():
    import quantized_selective_state_amd as ssdq
    inp, mu = _pair(90)
    note(f"correction: max |mu| {np.max(np.abs(mu)):.3e}, mean {np.mean(mu):.3e}")
    assert np.max(np.abs(mu)) > 0
    qx, sx, qB, sB, qC, sC = gpu_quantize_inputs(inp)
    dt, A, D, h0 = to_dev(inp["dt"]), to_dev(inp["A"]), to_dev(inp["D"]), to_dev(inp["h0"])
    y_c, h_c = ssdq.chunk_scan(qx, sx, qB, sB, qC, sC, dt, A, D, h0, chunk=inp["chunk"], y_corr=to_dev(mu))
    y_p, h_p = ssdq.chunk_scan(qx, sx, qB, sB, qC, sC, dt, A, D, h0, chunk=inp["chunk"])
    torch.cuda.synchronize()
    y_c, h_c = y_c.float().cpu().numpy(), h_c.cpu().numpy()
    y_p, h_p = y_p.float().cpu().numpy(), h_p.cpu().numpy()
    assert np.array_equal(h_c, h_p)                       # the state does not see the correction
    c = oracle.codes_from_inputs(inp)
    y_ref, h_ref, _ = oracle.ssd(c)
    ey, eh = rel_err(y_c, y_ref), rel_err(h_c, h_ref)
    note(f"corrected prefill: y_err={ey:.3e} h_err={eh:.3e}")
    assert ey <= Y_TOL and eh <= H_TOL
    # the corrected output differs from the plain one by the correction (up to fp16 rounding of y)
    d = y_c - y_p - mu[None, None]
    assert np.max(np.abs(d)) <= 2.0 ** -10 * np.max(np.abs(y_p)) + 1e-6
    # and its per-channel mean error against the unquantized scan is smaller
    vals = dict(x=inp["x16"].astype(np.float64), B=inp["B16"].astype(np.float64), C=inp["C16"].astype(np.float64),
                dt=inp["dt"], A=inp["A"], D=inp["D"], h0=inp["h0"])
    e_plain = np.zeros((c.H, c.P))
    e_corr = np.zeros((c.H, c.P))
    for b in range(c.batch):
        for h in range(c.H):
            y_fp, _ = oracle.ssd_values_one(vals, b, h)
            e_plain[h] += (y_fp - y_p[b, :, h]).sum(axis=0)
            e_corr[h] += (y_fp - y_c[b, :, h]).sum(axis=0)
    n = c.batch * c.L
    mp, mc = np.mean(np.abs(e_plain / n)), np.mean(np.abs(e_corr / n))
    note(f"mean |per-channel mean error| on the test draw: {mp:.3e} without, {mc:.3e} with the correction")
    assert mc < 0.5 * mp


@pytest.mark.parametrize("fmt", ["f32", "f16", "i8"])
def test_decode_corrected_against_the_oracle(fmt):
    import quantized_selective_state_amd as ssdq
    shape = workloads.DecodeShape(f"dcorr_{fmt}", 4, 8, 8, 64, 128, 2, 0.5)
    dec = workloads.make_decode(shape, seed_index=91)
    mu = np.random.default_rng(92).normal(0, 0.05, size=(8, 64)).astype(np.float32)
    sx, sB, sC = to_dev(dec["x_scale"]), to_dev(dec["B_scale"]), to_dev(dec["C_scale"])
    qx, qB, qC = ssdq.quantize(to_dev(dec["x16"]), sx), ssdq.quantize(to_dev(dec["B16"]), sB), \
        ssdq.quantize(to_dev(dec["C16"]), sC)
    dt, A, D, m = to_dev(dec["dt"]), to_dev(dec["A"]), to_dev(dec["D"]), to_dev(mu)
    c = oracle.decode_as_prefill(dec)
    c.y_corr = mu
    scale = None
    if fmt == "f32":
        state = to_dev(dec["state"])
    elif fmt == "f16":
        dec["state"] = dec["state"].astype(np.float16).astype(np.float32)
        c.h0 = dec["state"]
        state = to_dev(dec["state"]).half()
    else:
        q0, s0, _ = oracle.requantize_rows_i8(dec["state"].reshape(-1, 128).astype(np.float64))
        q0, s0 = q0.reshape(dec["state"].shape), s0.reshape(dec["state"].shape[:3])
        state, scale = to_dev(q0), to_dev(s0)
    T = dec["x16"].shape[0]
    ys = torch.empty((T,) + tuple(qx.shape[1:]), dtype=torch.float16, device=qx.device)
    for t in range(T):
        ssdq.state_update(state, qx[t], sx, qB[t], sB, qC[t], sC, dt[t], A, D, y=ys[t], state_scale=scale, y_corr=m)
    torch.cuda.synchronize()
    y = ys.float().cpu().numpy()
    if fmt == "i8":
        y_ref = np.stack([oracle.ssd_one_state_i8(c, b, h, q0, s0)[0] for b in range(c.batch) for h in range(c.H)])
        y_ref = y_ref.reshape(c.batch, c.H, T, c.P).transpose(2, 0, 1, 3)
    else:
        y_ref = np.swapaxes(oracle.ssd(c, state_f16=(fmt == "f16"))[0], 0, 1)
    ey = rel_err(y, y_ref)
    note(f"corrected decode ({fmt} state): y_err={ey:.3e}")
    assert ey <= Y_TOL
