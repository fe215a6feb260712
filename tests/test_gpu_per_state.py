"""GPU parity of the B and C scales per (group, state) (SSDi8 Table 10: per-P(N) together with
per-H(G)): the per-channel quantizer bit for bit, the prefill scan on both state plans and the
decode step in the three state formats, against the oracle with the same scales.

Draws: make_calibrated_pair with state_spread = 1 gives every state column of B and C its own
magnitude exp(N(0, 1)) (the case a scale per state is for), and the scales are the calibration
draw's absmax per (group, state) / 127.  The bars are the scan's (y within 2e-3, h within 1e-4 of
the largest reference value).  The prefill folds the product of the two scales of each state into
the B codes as a 16-bit fixed-point number relative to the group's largest product; the error
that adds to each term is at most 2^-9 of that largest product per C code unit, far inside the y
bar (the oracle takes the products exactly in fp64)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import H_TOL, Y_TOL, compare_full, dev, note, rel_err, to_dev

pytestmark = pytest.mark.gpu

ALL_F16 = np.arange(65536, dtype=np.uint16).view(np.float16)


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _pair(seed, batch=2, seqlen=320, nheads=8, headdim=64, dstate=128, ngroups=2, chunk=128, h0_std=0.1,
          x_dist="outlier_heads", spread=1.0, per_state=True, **kw):
    shape = workloads.PrefillShape(f"pn{seed}", batch, seqlen, nheads, headdim, dstate, ngroups, chunk,
                                   x_dist, "fixed_bias", h0_std)
    return workloads.make_calibrated_pair(shape, seed, bc_per_state=per_state, state_spread=spread, **kw)


def _gpu_scan(inp, with_D=True, with_h0=True, y_corr=None):
    import quantized_selective_state_amd as ssdq
    sx, sB, sC = to_dev(inp["x_scale"]), to_dev(inp["B_scale"]), to_dev(inp["C_scale"])
    qx, qB, qC = ssdq.quantize(to_dev(inp["x16"]), sx), ssdq.quantize(to_dev(inp["B16"]), sB), \
        ssdq.quantize(to_dev(inp["C16"]), sC)
    D = to_dev(inp["D"]) if with_D else None
    h0 = to_dev(inp["h0"]) if with_h0 else None
    y, hf = ssdq.chunk_scan(qx, sx, qB, sB, qC, sC, to_dev(inp["dt"]), to_dev(inp["A"]), D, h0,
                            chunk=inp["chunk"], y_corr=None if y_corr is None else to_dev(y_corr))
    torch.cuda.synchronize()
    codes = dict(qx=qx.cpu().numpy(), qB=qB.cpu().numpy(), qC=qC.cpu().numpy())
    return codes, y.float().cpu().numpy(), hf.cpu().numpy()


def _check(inp, with_D=True, with_h0=True, tag="", fused=None):
    import quantized_selective_state_amd as ssdq
    if fused is not None:
        assert ssdq.chunk_scan_state_fused(inp["batch"], inp["nheads"]) == fused
    assert inp["B_scale"].shape == (inp["ngroups"], inp["dstate"])
    codes, y, hf = _gpu_scan(inp, with_D, with_h0, inp.get("y_corr"))
    c = oracle.codes_from_inputs(inp)
    assert c.per_state
    if not with_D:
        c.D = None
    if not with_h0:
        c.h0 = None
    assert np.array_equal(codes["qx"], c.qx) and np.array_equal(codes["qB"], c.qB) \
        and np.array_equal(codes["qC"], c.qC)
    y_ref, h_ref, _ = oracle.ssd(c)
    ey, eh = rel_err(y, y_ref), rel_err(hf, h_ref)
    note(f"per-state {tag}: y_err={ey:.3e} h_err={eh:.3e}")
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(hf))
    assert ey <= Y_TOL, ey
    assert eh <= H_TOL, eh
    return y


@pytest.mark.parametrize("inner", [64, 16, 5])     # vector path (16 per thread) and scalar path
def test_quantize_every_f16_value(inner):
    import quantized_selective_state_amd as ssdq
    nscale = 3
    rng = np.random.default_rng(60 + inner)
    scale = np.exp2(rng.uniform(-20, 6, size=(nscale, inner))).astype(np.float32)
    scale.flat[:4] = [1.0, 1.0 / 127.0, 0.8160377, 37.5]
    n = 65536 - 65536 % inner
    x = np.ascontiguousarray(np.repeat(ALL_F16[:n].reshape(n // inner, 1, inner), nscale, axis=1))
    note(f"per-channel quantize exhaustive inner={inner} shape={x.shape}")
    got = ssdq.quantize(to_dev(x), to_dev(scale)).cpu().numpy()
    ref = oracle.quantize_per_channel(x, scale)
    bad = np.count_nonzero(got != ref)
    assert bad == 0, f"{bad} code mismatches"


def test_quantize_workload_tensors():
    import quantized_selective_state_amd as ssdq
    _, inp = _pair(61, batch=2, seqlen=512, nheads=8, ngroups=4)
    for key, skey in (("B16", "B_scale"), ("C16", "C_scale")):
        got = ssdq.quantize(to_dev(inp[key]), to_dev(inp[skey])).cpu().numpy()
        ref = oracle.quantize_per_channel(inp[key], inp[skey])
        assert np.array_equal(got, ref), f"{key}: {np.count_nonzero(got != ref)} mismatches"
        # the test draw exceeds the calibrated range in places: codes saturate at +-127
        assert np.abs(got.astype(np.int32)).max() == 127


@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_prefill_three_kernel_plan(chunk):
    _, inp = _pair(62, chunk=chunk)
    _check(inp, tag=f"three-kernel chunk={chunk}", fused=False)


@pytest.mark.parametrize("chunk", [64, 256])
def test_prefill_fused_plan(chunk):
    nheads = 64
    _, inp = _pair(63, batch=-(-_cus() // nheads), seqlen=300, nheads=nheads, headdim=32, dstate=64, chunk=chunk)
    _check(inp, tag=f"fused chunk={chunk}", fused=True)


@pytest.mark.parametrize("L,Q,P,N,G", [(250, 64, 16, 16, 1), (129, 128, 64, 80, 2), (65, 64, 48, 48, 4),
                                       (1, 64, 32, 128, 2)])
def test_prefill_ragged_lengths_and_dims(L, Q, P, N, G):
    _, inp = _pair(64, batch=2, seqlen=L, nheads=4, headdim=P, dstate=N, ngroups=G, chunk=Q, h0_std=0.2)
    _check(inp, tag=f"L={L} Q={Q} P={P} N={N} G={G}")


def test_prefill_without_D_and_h0():
    _, inp = _pair(65, seqlen=200, nheads=4, headdim=16, dstate=32, ngroups=4, chunk=64, h0_std=0.3)
    _check(inp, with_D=False, with_h0=False, tag="no D, no h0")
    _check(inp, with_D=False, with_h0=True, tag="no D, h0")


def test_prefill_uniform_state_scales_equal_the_group_scales():
    # every state of a group on the same scale: the per-state call computes what the per-group
    # call does (the fixed-point products are then exact: each is the group's largest)
    import quantized_selective_state_amd as ssdq
    _, inp = _pair(66, spread=0.0, per_state=False)
    _, y_g, h_g = _gpu_scan(inp)
    G, N = inp["ngroups"], inp["dstate"]
    inp_ps = dict(inp, B_scale=np.repeat(inp["B_scale"][:, None], N, axis=1),
                  C_scale=np.repeat(inp["C_scale"][:, None], N, axis=1))
    y_ps = _check(inp_ps, tag="uniform states")
    assert rel_err(y_ps, y_g) <= 2.0 ** -10, rel_err(y_ps, y_g)
    assert ssdq is not None


def test_prefill_with_correction_and_percentile_clipping():
    # one-sided x with the x scales clipped at the 90th percentile (many saturated codes), the
    # per-state B/C scales, and the mean correction calibrated on the calibration draw
    cal, inp = _pair(67, x_mean=0.5, x_clip_pct=90.0)
    mu = oracle.mean_correction(cal)
    assert np.max(np.abs(mu)) > 0
    inp["y_corr"] = mu
    c = oracle.codes_from_inputs(inp)
    sat = np.mean(np.abs(c.qx.astype(np.int32)) == 127)
    note(f"saturated x codes: {sat:.3%}")
    assert sat > 0.01
    _check(inp, tag="corrected + clipped")


def test_per_state_scales_reduce_the_error_on_spread_states():
    # the same draws quantized with one scale per group and with one per (group, state): against
    # the unquantized scan (fp64 over the fp16 values) the per-state output is closer
    _, grp = _pair(68, batch=1, seqlen=256, nheads=4, per_state=False)
    _, pst = _pair(68, batch=1, seqlen=256, nheads=4, per_state=True)
    assert np.array_equal(grp["B16"], pst["B16"])
    _, y_g, _ = _gpu_scan(grp)
    _, y_p, _ = _gpu_scan(pst)
    vals = dict(x=pst["x16"].astype(np.float64), B=pst["B16"].astype(np.float64),
                C=pst["C16"].astype(np.float64), dt=pst["dt"], A=pst["A"], D=pst["D"], h0=pst["h0"])
    y_fp = np.stack([oracle.ssd_values_one(vals, 0, h)[0] for h in range(pst["nheads"])], axis=1)
    eg, ep = rel_err(y_g[0], y_fp), rel_err(y_p[0], y_fp)
    note(f"error against the unquantized scan: per group {eg:.3e}, per state {ep:.3e}")
    assert ep < eg


def test_full_size_fused_workload():
    # the 1.3B prefill shape (4 x 2048 tokens, 64 heads of 64, 128 states, fused plan) with
    # per-state scales, every sequence against the oracle
    s = workloads.WORKLOADS["mamba2-1.3b-prefill"]
    _, inp = _pair(69, batch=s.batch, seqlen=s.seqlen, nheads=s.nheads, headdim=s.headdim, dstate=s.dstate,
                   ngroups=s.ngroups, chunk=s.chunk, h0_std=0.1)
    _, y, hf = _gpu_scan(inp)
    c = oracle.codes_from_inputs(inp)
    compare_full(c, lambda b: y[b], lambda b: hf[b], "per-state mamba2-1.3b-prefill")


def _as_decode(inp):
    sw = lambda a: np.ascontiguousarray(np.swapaxes(a, 0, 1))
    return dict(state=inp["h0"], x16=sw(inp["x16"]), B16=sw(inp["B16"]), C16=sw(inp["C16"]), dt=sw(inp["dt"]),
                A=inp["A"], D=inp["D"], x_scale=inp["x_scale"], B_scale=inp["B_scale"], C_scale=inp["C_scale"],
                batch=inp["batch"], steps=inp["seqlen"], nheads=inp["nheads"], headdim=inp["headdim"],
                dstate=inp["dstate"], ngroups=inp["ngroups"])


@pytest.mark.parametrize("fmt", ["f32", "f16", "i8"])
@pytest.mark.parametrize("N,G,corr", [(128, 2, False), (64, 8, True), (64, 1, False)])
def test_decode_against_the_oracle(fmt, N, G, corr):
    import quantized_selective_state_amd as ssdq
    _, inp = _pair(70 + N + G + int(corr), batch=3, seqlen=8, nheads=8, headdim=64, dstate=N, ngroups=G, h0_std=0.5)
    dec = _as_decode(inp)
    mu = np.random.default_rng(71).normal(0, 0.05, size=(8, 64)).astype(np.float32) if corr else None
    sx, sB, sC = to_dev(dec["x_scale"]), to_dev(dec["B_scale"]), to_dev(dec["C_scale"])
    qx, qB, qC = ssdq.quantize(to_dev(dec["x16"]), sx), ssdq.quantize(to_dev(dec["B16"]), sB), \
        ssdq.quantize(to_dev(dec["C16"]), sC)
    dt, A, D = to_dev(dec["dt"]), to_dev(dec["A"]), to_dev(dec["D"])
    c = oracle.decode_as_prefill(dec)
    assert c.per_state
    c.y_corr = mu
    scale = None
    if fmt == "f32":
        state = to_dev(dec["state"])
    elif fmt == "f16":
        dec["state"] = dec["state"].astype(np.float16).astype(np.float32)
        c.h0 = dec["state"]
        state = to_dev(dec["state"]).half()
    else:
        q0, s0, _ = oracle.requantize_rows_i8(dec["state"].reshape(-1, N).astype(np.float64))
        q0, s0 = q0.reshape(dec["state"].shape), s0.reshape(dec["state"].shape[:3])
        state, scale = to_dev(q0), to_dev(s0)
    T = dec["x16"].shape[0]
    ys = torch.empty((T,) + tuple(qx.shape[1:]), dtype=torch.float16, device=dev())
    m = None if mu is None else to_dev(mu)
    for t in range(T):
        ssdq.state_update(state, qx[t], sx, qB[t], sB, qC[t], sC, dt[t], A, D, y=ys[t], state_scale=scale, y_corr=m)
    torch.cuda.synchronize()
    y = ys.float().cpu().numpy()
    if fmt == "i8":
        y_ref = np.stack([oracle.ssd_one_state_i8(c, b, h, q0, s0)[0] for b in range(c.batch) for h in range(c.H)])
        y_ref = y_ref.reshape(c.batch, c.H, T, c.P).transpose(2, 0, 1, 3)
    else:
        y_ref, h_ref, _ = oracle.ssd(c, state_f16=(fmt == "f16"))
        y_ref = np.swapaxes(y_ref, 0, 1)
        h = state.float().cpu().numpy()
        eh = rel_err(h, h_ref)
        note(f"per-state decode ({fmt}, N={N}, G={G}): h_err={eh:.3e}")
        # binary16 cache: a few spacings (2^-10 of a value) where the fp32 and the exact update
        # round to different neighbours
        assert eh <= (4 * 2.0 ** -10 if fmt == "f16" else H_TOL)
    ey = rel_err(y, y_ref)
    note(f"per-state decode ({fmt}, N={N}, G={G}, corr={corr}): y_err={ey:.3e}")
    assert ey <= Y_TOL
