"""GPU parity of the four-wave form of the folded state kernel (ssdq_chunk_scan_plan == 4: many
more (batch, head) sequences than CUs, two blocks of four waves per CU, each wave one channel tile
over all tokens and states).  Every sequence of each shape is compared with the oracle at the
scan's bars; the carried state in the workspace is checked against the oracle's chunk-boundary
states; the shapes cover the three chunk sizes, ragged lengths, narrow heads, a partial 64-state
block, x scales per (head, channel), B and C scales per (group, state), all scale layouts with
the output correction, and an in-place final state."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import (H_TOL, Y_TOL, carried_state, compare_full, dev, gpu_quantize_inputs, note, oracle_codes,
                      rel_err, to_dev)

pytestmark = pytest.mark.gpu


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _shape_for_plan4(nheads):
    """A batch with 2 sequences per CU (the four-wave plan's best case)."""
    return max(1, -(-2 * _cus() // nheads))


def _make(seed, nheads=64, seqlen=300, headdim=64, dstate=128, ngroups=2, chunk=128, h0_std=0.2, **kw):
    batch = _shape_for_plan4(nheads)
    return workloads.make_custom_prefill(seed, batch=batch, seqlen=seqlen, nheads=nheads, headdim=headdim,
                                         dstate=dstate, ngroups=ngroups, chunk=chunk, h0_std=h0_std, **kw)


def _run(inp, y_corr=None, layout=0, h_inplace=False):
    import quantized_selective_state_amd as ssdq
    qx, sx, qB, sB, qC, sC = gpu_quantize_inputs(inp)
    h0 = to_dev(inp["h0"]) if inp.get("h0") is not None else None
    hf = h0 if h_inplace else None
    y, hf = ssdq.chunk_scan(qx, sx, qB, sB, qC, sC, to_dev(inp["dt"]), to_dev(inp["A"]), to_dev(inp["D"]), h0,
                            chunk=inp["chunk"], h_final=hf, y_corr=None if y_corr is None else to_dev(y_corr))
    torch.cuda.synchronize()
    return y, hf


def _check(inp, tag, plan=4, y_corr=None, h_inplace=False):
    import quantized_selective_state_amd as ssdq
    layout = (ssdq.SCALES_X_PER_CHANNEL if np.ndim(inp["x_scale"]) == 2 else 0) | (
        ssdq.SCALES_BC_PER_STATE if np.ndim(inp["B_scale"]) == 2 else 0)
    assert ssdq.chunk_scan_plan(inp["batch"], inp["nheads"], layout) == plan
    y, hf = _run(inp, y_corr, layout, h_inplace)
    c = oracle.codes_from_inputs(inp)
    c.y_corr = y_corr
    note(f"plan-4 {tag}: b={inp['batch']} H={inp['nheads']} L={inp['seqlen']} Q={inp['chunk']}")
    yh, hh = y.float().cpu().numpy(), hf.cpu().numpy()
    compare_full(c, lambda b: yh[b], lambda b: hh[b], f"plan-4 {tag}")


@pytest.mark.parametrize("chunk,seqlen", [(64, 250), (128, 300), (256, 333)])
def test_chunk_sizes_and_ragged_lengths(chunk, seqlen):
    _check(_make(110 + chunk, chunk=chunk, seqlen=seqlen), f"Q={chunk} L={seqlen}")


@pytest.mark.parametrize("chunk,seqlen", [(64, 700), (128, 1100), (256, 1300)])
def test_many_chunks(chunk, seqlen):
    # 11, 9 and 6 chunks: the chunk weights go through both LDS slots (prepared one group of four
    # chunks ahead) and the staged units through both tile buffers more than once; at chunk 256
    # the last chunk's second 128-token unit lies wholly past the sequence end
    _check(_make(140 + chunk, chunk=chunk, seqlen=seqlen, h0_std=0.1), f"Q={chunk} L={seqlen}")


@pytest.mark.parametrize("P,N,G", [(16, 16, 1), (32, 80, 4), (48, 64, 8)])
def test_head_and_state_widths(P, N, G):
    _check(_make(120 + P + N, headdim=P, dstate=N, ngroups=G, seqlen=200), f"P={P} N={N} G={G}")


def test_channel_scales_and_correction():
    import quantized_selective_state_amd as ssdq
    nheads = 64
    shape = workloads.PrefillShape("p4pc", _shape_for_plan4(nheads), 256, nheads, 64, 128, 2, 128, "outlier_heads",
                                   "fixed_bias", 0.1)
    cal, inp = workloads.make_calibrated_pair(shape, 130, channel_spread=1.0, x_clusters=8)
    mu = oracle.mean_correction(cal)
    assert ssdq.chunk_scan_plan(inp["batch"], nheads, ssdq.SCALES_X_PER_CHANNEL) == 4
    _check(inp, "x per channel + correction", y_corr=mu)


@pytest.mark.parametrize("chunk", [128, 256])
def test_state_scales(chunk):
    # B, C scales per (group, state): the per-state factors of the update come from LDS
    nheads = 64
    shape = workloads.PrefillShape("p4ps", _shape_for_plan4(nheads), 300, nheads, 64, 128, 2, chunk, "outlier_heads",
                                   "fixed_bias", 0.1)
    _, inp = workloads.make_calibrated_pair(shape, 131, bc_per_state=True, state_spread=1.0)
    _check(inp, f"B, C per state, Q={chunk}")


def test_all_scale_layouts_with_correction():
    nheads = 64
    shape = workloads.PrefillShape("p4all", _shape_for_plan4(nheads), 256, nheads, 32, 64, 4, 64, "outlier_heads",
                                   "fixed_bias", 0.2)
    cal, inp = workloads.make_calibrated_pair(shape, 134, bc_per_state=True, state_spread=1.0, channel_spread=1.0,
                                              x_clusters=4)
    _check(inp, "x per channel + B, C per state + correction", y_corr=oracle.mean_correction(cal))


def test_final_state_in_place():
    _check(_make(132, seqlen=200), "h_final aliases h0", h_inplace=True)


def test_carried_state_in_the_workspace():
    import quantized_selective_state_amd as ssdq
    inp = _make(133, nheads=64, seqlen=300, chunk=128)
    qx, sx, qB, sB, qC, sC = gpu_quantize_inputs(inp)
    buf = ssdq.ScanBuffers(qx, sx, qB, sB, qC, sC, to_dev(inp["dt"]), to_dev(inp["A"]), to_dev(inp["D"]),
                           to_dev(inp["h0"]), chunk=128)
    assert ssdq.chunk_scan_plan(inp["batch"], inp["nheads"]) == 4
    buf.run_stage(0)
    torch.cuda.synchronize()
    views = buf.workspace_views()
    Hprev = carried_state(views["hprev"].cpu().numpy(), views["hscale"].cpu().numpy())
    c = oracle_codes(inp)
    for b in (0, inp["batch"] - 1):
        _, _, bounds = oracle.ssd(c, pairs=[(b, h) for h in range(c.H)], chunk=128)
        assert rel_err(Hprev[b], bounds[b]) <= 1e-4, rel_err(Hprev[b], bounds[b])
