"""GPU parity of x scales per (head, channel) -- the static scales that Quamba2's sort-and-cluster
of the x channels leaves behind (one per channel cluster, given as a (H, P) table): the quantizer
bit for bit, the prefill scan on both state plans (alone, with B and C scales per (group, state),
with the output correction) and the decode step in the three state formats, against the oracle
with the same scales.

Draws: make_calibrated_pair with channel_spread = 1 gives every x channel of every head its own
magnitude exp(N(0, 1)), and the x scales come from k channel clusters of the calibration draw
(cluster_channel_scales).  The bars are the scan's (y within 2e-3, h within 1e-4 of the largest
reference value): the kernels apply each channel's scale in fp32 where the per-head call applies
the head's."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import H_TOL, Y_TOL, compare_full, dev, note, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _pair(seed, batch=2, seqlen=320, nheads=8, headdim=64, dstate=128, ngroups=2, chunk=128, h0_std=0.1,
          x_dist="outlier_heads", spread=1.0, clusters=4, per_state=False, **kw):
    shape = workloads.PrefillShape(f"pc{seed}", batch, seqlen, nheads, headdim, dstate, ngroups, chunk,
                                   x_dist, "fixed_bias", h0_std)
    return workloads.make_calibrated_pair(shape, seed, channel_spread=spread, x_clusters=clusters,
                                          bc_per_state=per_state, state_spread=1.0 if per_state else 0.0, **kw)


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
    assert inp["x_scale"].shape == (inp["nheads"], inp["headdim"])
    codes, y, hf = _gpu_scan(inp, with_D, with_h0, inp.get("y_corr"))
    c = oracle.codes_from_inputs(inp)
    assert c.x_per_channel
    if not with_D:
        c.D = None
    if not with_h0:
        c.h0 = None
    assert np.array_equal(codes["qx"], c.qx) and np.array_equal(codes["qB"], c.qB) \
        and np.array_equal(codes["qC"], c.qC)
    y_ref, h_ref, _ = oracle.ssd(c)
    ey, eh = rel_err(y, y_ref), rel_err(hf, h_ref)
    note(f"per-channel x {tag}: y_err={ey:.3e} h_err={eh:.3e}")
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(hf))
    assert ey <= Y_TOL, ey
    assert eh <= H_TOL, eh
    return y, hf


def test_quantize_x_with_channel_scales():
    import quantized_selective_state_amd as ssdq
    _, inp = _pair(81, batch=2, seqlen=512)
    got = ssdq.quantize(to_dev(inp["x16"]), to_dev(inp["x_scale"])).cpu().numpy()
    ref = oracle.quantize_per_channel(inp["x16"], inp["x_scale"])
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} mismatches"


@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_prefill_three_kernel_plan(chunk):
    _, inp = _pair(82, chunk=chunk)
    _check(inp, tag=f"three-kernel chunk={chunk}", fused=False)


@pytest.mark.parametrize("chunk,clusters", [(64, 64), (256, 4)])
def test_prefill_fused_plan(chunk, clusters):
    nheads = 64
    _, inp = _pair(83, batch=-(-_cus() // nheads), seqlen=300, nheads=nheads, headdim=32, dstate=64, chunk=chunk,
                   clusters=min(clusters, 32))
    _check(inp, tag=f"fused chunk={chunk} clusters={clusters}", fused=True)


@pytest.mark.parametrize("L,Q,P,N,G", [(250, 64, 16, 16, 1), (129, 128, 64, 80, 2), (1, 64, 32, 128, 2)])
def test_prefill_ragged_lengths_and_dims(L, Q, P, N, G):
    _, inp = _pair(84, batch=2, seqlen=L, nheads=4, headdim=P, dstate=N, ngroups=G, chunk=Q, h0_std=0.2,
                   clusters=min(4, P))
    _check(inp, tag=f"L={L} Q={Q} P={P} N={N} G={G}")


def test_prefill_without_D_and_h0():
    _, inp = _pair(85, seqlen=200, nheads=4, headdim=16, dstate=32, ngroups=4, chunk=64, h0_std=0.3, clusters=2)
    _check(inp, with_D=False, with_h0=False, tag="no D, no h0")


@pytest.mark.parametrize("fused", [False, True])
def test_prefill_with_state_scales_and_correction(fused):
    # every scale layout bit at once, with the mean correction calibrated on the calibration draw
    nheads = 64 if fused else 8
    batch = -(-_cus() // nheads) if fused else 2
    cal, inp = _pair(86, batch=batch, seqlen=256, nheads=nheads, headdim=32, dstate=64, chunk=128, per_state=True)
    inp["y_corr"] = oracle.mean_correction(cal)
    assert np.max(np.abs(inp["y_corr"])) > 0
    _check(inp, tag=f"per-state B/C + correction, fused={fused}", fused=fused)


def test_constant_channel_scales_match_the_per_head_call():
    # one cluster: every channel of a head on the head's scale; the per-channel call then computes
    # what the per-head call does, up to where the scale is applied
    _, inp = _pair(87, spread=0.0, clusters=1)
    head = dict(inp, x_scale=np.ascontiguousarray(inp["x_scale"][:, 0]))
    _, y_h, h_h = _gpu_scan(head)
    y_c, h_c = _check(inp, tag="one cluster")
    assert rel_err(y_c, y_h) <= 2.0 ** -10, rel_err(y_c, y_h)
    assert rel_err(h_c, h_h) <= 1e-6, rel_err(h_c, h_h)


def test_channel_clusters_reduce_the_error_on_spread_channels():
    # the same draw quantized with one x scale per head and with one per (head, channel cluster):
    # against the unquantized scan (fp64 over the fp16 values) the clustered output is closer in
    # the root-mean-square sense (finer steps on every small channel).  Its largest single error
    # need not be: a channel whose test values exceed its calibrated range saturates, which a
    # head-wide scale (set by the head's largest channel) rarely lets happen.
    _, hd = _pair(88, batch=1, seqlen=256, nheads=4, clusters=1)
    _, cl = _pair(88, batch=1, seqlen=256, nheads=4, clusters=8)
    assert np.array_equal(hd["x16"], cl["x16"])
    _, y_h, _ = _gpu_scan(hd)
    _, y_c, _ = _gpu_scan(cl)
    vals = dict(x=cl["x16"].astype(np.float64), B=cl["B16"].astype(np.float64),
                C=cl["C16"].astype(np.float64), dt=cl["dt"], A=cl["A"], D=cl["D"], h0=cl["h0"])
    y_fp = np.stack([oracle.ssd_values_one(vals, 0, h)[0] for h in range(cl["nheads"])], axis=1)
    rms = lambda y: float(np.sqrt(np.mean((y - y_fp) ** 2) / np.mean(y_fp ** 2)))
    eh, ec = rms(y_h[0]), rms(y_c[0])
    note(f"rms error against the unquantized scan: per head {eh:.3e}, 8 channel clusters {ec:.3e}")
    assert ec < 0.8 * eh


def test_full_size_fused_workload():
    # the 1.3B prefill shape with per-(head, channel) x scales from 8 clusters, every sequence
    s = workloads.WORKLOADS["mamba2-1.3b-prefill"]
    _, inp = _pair(89, batch=s.batch, seqlen=s.seqlen, nheads=s.nheads, headdim=s.headdim, dstate=s.dstate,
                   ngroups=s.ngroups, chunk=s.chunk, h0_std=0.1, clusters=8)
    _, y, hf = _gpu_scan(inp)
    c = oracle.codes_from_inputs(inp)
    assert c.x_per_channel
    compare_full(c, lambda b: y[b], lambda b: hf[b], "per-channel x mamba2-1.3b-prefill")


def _as_decode(inp):
    sw = lambda a: np.ascontiguousarray(np.swapaxes(a, 0, 1))
    return dict(state=inp["h0"], x16=sw(inp["x16"]), B16=sw(inp["B16"]), C16=sw(inp["C16"]), dt=sw(inp["dt"]),
                A=inp["A"], D=inp["D"], x_scale=inp["x_scale"], B_scale=inp["B_scale"], C_scale=inp["C_scale"],
                batch=inp["batch"], steps=inp["seqlen"], nheads=inp["nheads"], headdim=inp["headdim"],
                dstate=inp["dstate"], ngroups=inp["ngroups"])


@pytest.mark.parametrize("fmt", ["f32", "f16", "i8"])
@pytest.mark.parametrize("N,G,per_state,corr", [(128, 2, False, False), (64, 8, True, True), (64, 1, False, True)])
def test_decode_against_the_oracle(fmt, N, G, per_state, corr):
    import quantized_selective_state_amd as ssdq
    _, inp = _pair(90 + N + G + int(corr), batch=3, seqlen=8, nheads=8, headdim=64, dstate=N, ngroups=G,
                   h0_std=0.5, per_state=per_state)
    dec = _as_decode(inp)
    mu = np.random.default_rng(91).normal(0, 0.05, size=(8, 64)).astype(np.float32) if corr else None
    sx, sB, sC = to_dev(dec["x_scale"]), to_dev(dec["B_scale"]), to_dev(dec["C_scale"])
    qx, qB, qC = ssdq.quantize(to_dev(dec["x16"]), sx), ssdq.quantize(to_dev(dec["B16"]), sB), \
        ssdq.quantize(to_dev(dec["C16"]), sC)
    dt, A, D = to_dev(dec["dt"]), to_dev(dec["A"]), to_dev(dec["D"])
    c = oracle.decode_as_prefill(dec)
    assert c.x_per_channel and c.per_state == int(per_state)
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
        note(f"per-channel x decode ({fmt}, N={N}, G={G}): h_err={eh:.3e}")
        assert eh <= (4 * 2.0 ** -10 if fmt == "f16" else H_TOL)
    ey = rel_err(y, y_ref)
    note(f"per-channel x decode ({fmt}, N={N}, G={G}, per_state={per_state}, corr={corr}): y_err={ey:.3e}")
    assert ey <= Y_TOL
