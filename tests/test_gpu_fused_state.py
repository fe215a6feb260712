"""GPU parity of the prefill path in which stage 0 carries the state across chunks itself
(one block per (batch, head) sequence, used when there are at least as many sequences as
CUs): y, h_final and the workspace intermediates it writes (Acs, carried state) against the
fp64 oracle, at sizes the oracle finishes in seconds, with ragged tails and edge cases.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import (H_TOL, Y_TOL, carried_state, gpu_prefill, gpu_quantize_inputs, note, oracle_codes, rel_err,
                      to_dev)

pytestmark = pytest.mark.gpu


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _fused_inputs(seed, seqlen, headdim, dstate, ngroups, chunk, h0_std=0.1, x_dist="outlier_heads"):
    """Enough (batch, head) sequences for the folded path on this device (>= #CUs)."""
    nheads = 64
    batch = -(-_cus() // nheads)
    return workloads.make_custom_prefill(seed, batch=batch, seqlen=seqlen, nheads=nheads, headdim=headdim,
                                         dstate=dstate, ngroups=ngroups, chunk=chunk, x_dist=x_dist,
                                         h0_std=h0_std)


def _check(inp, with_D=True, with_h0=True, tag=""):
    import quantized_selective_state_amd as ssdq
    assert ssdq.chunk_scan_state_fused(inp["batch"], inp["nheads"])
    codes, y, hf = gpu_prefill(inp, None, with_D, with_h0)
    c = oracle_codes(inp, with_D, with_h0)
    assert np.array_equal(codes["qx"], c.qx)
    y_ref, h_ref, _ = oracle.ssd(c)
    ey, eh = rel_err(y, y_ref), rel_err(hf, h_ref)
    note(f"{tag} y_err={ey:.3e} h_err={eh:.3e}")
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(hf))
    assert ey <= Y_TOL, ey
    assert eh <= H_TOL, eh


def test_plan_follows_cu_count():
    import quantized_selective_state_amd as ssdq
    n = _cus()
    assert ssdq.chunk_scan_state_fused(1, n) and ssdq.chunk_scan_state_fused(n, 1)
    assert not ssdq.chunk_scan_state_fused(1, n - 1)
    assert not ssdq.chunk_scan_state_fused(0, 4) and not ssdq.chunk_scan_state_fused(4, -1)


@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_chunk_sizes(chunk):
    _check(_fused_inputs(31, 512, 32, 64, 2, chunk), tag=f"fused chunk={chunk}")


@pytest.mark.parametrize("L,Q", [(1, 64), (200, 64), (300, 128), (700, 256)])
def test_ragged_lengths(L, Q):
    _check(_fused_inputs(32, L, 16, 32, 4, Q, h0_std=0.3), tag=f"fused L={L} Q={Q}")


@pytest.mark.parametrize("P,N", [(16, 16), (64, 128), (48, 80)])
def test_head_and_state_dims(P, N):
    _check(_fused_inputs(33, 384, P, N, 1, 128), tag=f"fused P={P} N={N}")


def test_without_D_and_h0():
    inp = _fused_inputs(34, 256, 32, 32, 8, 64, h0_std=0.2)
    _check(inp, with_D=False, with_h0=False, tag="fused no D, no h0")
    _check(inp, with_D=True, with_h0=False, tag="fused D, no h0")


def test_no_decay_and_decay_to_zero():
    inp = _fused_inputs(35, 320, 16, 32, 1, 64, h0_std=0.1)
    inp["A"] = np.zeros_like(inp["A"])
    _check(inp, tag="fused A=0")
    inp["A"] = np.full_like(inp["A"], -1e5)
    _check(inp, tag="fused A=-1e5")


def test_h_final_may_alias_h0():
    import quantized_selective_state_amd as ssdq
    inp = _fused_inputs(36, 256, 32, 32, 1, 64, h0_std=0.2)
    qx, sx, qB, sB, qC, sC = gpu_quantize_inputs(inp)
    h = to_dev(inp["h0"])
    y, _ = ssdq.chunk_scan(qx, sx, qB, sB, qC, sC, to_dev(inp["dt"]), to_dev(inp["A"]), to_dev(inp["D"]), h,
                           chunk=64, h_final=h)
    c = oracle_codes(inp)
    y_ref, h_ref, _ = oracle.ssd(c)
    assert rel_err(h.cpu().numpy(), h_ref) <= H_TOL
    assert rel_err(y.float().cpu().numpy(), y_ref) <= Y_TOL


def test_intermediates():
    """Stage 0 writes Acs and the carried state; stage 1 changes nothing."""
    import quantized_selective_state_amd as ssdq
    inp = _fused_inputs(37, 600, 64, 128, 2, 256)
    qx, sx, qB, sB, qC, sC = gpu_quantize_inputs(inp)
    buf = ssdq.ScanBuffers(qx, sx, qB, sB, qC, sC, to_dev(inp["dt"]), to_dev(inp["A"]), to_dev(inp["D"]),
                           to_dev(inp["h0"]), chunk=256)
    views = buf.workspace_views()
    buf.run_stage(0)
    torch.cuda.synchronize()
    acs = views["acs"].cpu().numpy()
    limbs0 = views["hprev"].cpu().numpy().copy()
    hs0 = views["hscale"].cpu().numpy().copy()
    buf.run_stage(1)
    torch.cuda.synchronize()
    assert np.array_equal(limbs0, views["hprev"].cpu().numpy()) and np.array_equal(hs0, views["hscale"].cpu().numpy())
    buf.run_stage(2)
    torch.cuda.synchronize()
    c = oracle_codes(inp)
    pairs = [(0, 0), (0, 5), (1, 17), (inp["batch"] - 1, 63)]
    _, h_ref, bounds = oracle.ssd(c, pairs=pairs, chunk=256)
    Hprev = carried_state(limbs0, hs0)
    for b, h in pairs:
        a_ref = oracle.chunk_cumsum(c, b, h, 256)
        valid = np.isfinite(a_ref)
        assert np.max(np.abs(acs[b, h][valid] - a_ref[valid])) <= 2e-5 * max(1.0, np.max(np.abs(a_ref[valid])))
        assert rel_err(Hprev[b, :, h], bounds[b, :, h]) <= 1e-4
        assert rel_err(buf.h_final[b, h].cpu().numpy(), h_ref[b, h]) <= H_TOL
