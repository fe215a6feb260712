"""GPU parity of ssdq_chunk_scan (prefill) against the fp64 oracle.

Bar (stated for the scan): codes bit-exact; max|y - y_ref| <= 2e-3 max|y_ref| and
max|h_final - h_ref| <= 1e-4 max|h_ref| over the whole output tensors.  Full-size
workloads run the whole GPU path at their real shape and compare every (batch,
head) sequence, streamed one batch index at a time.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import (H_TOL, Y_TOL, carried_state, dev, gpu_prefill, gpu_quantize_inputs, note, oracle_codes,
                      compare_full, rel_err, to_dev)

pytestmark = pytest.mark.gpu


def _check_full(inp, chunk=None, with_D=True, with_h0=True, tag=""):
    codes, y, hf = gpu_prefill(inp, chunk, with_D, with_h0)
    c = oracle_codes(inp, with_D, with_h0)
    assert np.array_equal(codes["qx"], c.qx) and np.array_equal(codes["qB"], c.qB) \
        and np.array_equal(codes["qC"], c.qC)
    y_ref, h_ref, _ = oracle.ssd(c)
    ey, eh = rel_err(y, y_ref), rel_err(hf, h_ref)
    note(f"{tag} y_err={ey:.3e} h_err={eh:.3e}")
    assert ey <= Y_TOL, ey
    assert eh <= H_TOL, eh
    return ey, eh


def test_tiny_workload():
    _check_full(workloads.make_prefill("tiny"), tag="tiny")


@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_chunk_size_invariance(chunk):
    inp = workloads.make_custom_prefill(11, batch=2, seqlen=512, nheads=4, headdim=64, dstate=128, ngroups=2,
                                        chunk=chunk, x_dist="outlier_heads", h0_std=0.1)
    _check_full(inp, tag=f"chunk={chunk}")


@pytest.mark.parametrize("L,Q", [(250, 64), (1, 64), (65, 64), (300, 256), (129, 128)])
def test_ragged_lengths(L, Q):
    inp = workloads.make_custom_prefill(12, batch=2, seqlen=L, nheads=4, headdim=32, dstate=32, ngroups=2, chunk=Q,
                                        h0_std=0.2)
    _check_full(inp, tag=f"L={L} Q={Q}")


@pytest.mark.parametrize("P,N", [(16, 16), (48, 48), (64, 64), (32, 128), (64, 80)])
def test_head_and_state_dims(P, N):
    inp = workloads.make_custom_prefill(13, batch=1, seqlen=320, nheads=3, headdim=P, dstate=N, ngroups=1,
                                        chunk=64, h0_std=0.1)
    _check_full(inp, tag=f"P={P} N={N}")


def test_without_D_and_h0():
    inp = workloads.make_custom_prefill(14, batch=2, seqlen=200, nheads=4, headdim=16, dstate=32, ngroups=4,
                                        chunk=64, h0_std=0.3)
    _check_full(inp, with_D=False, with_h0=False, tag="no D, no h0")
    _check_full(inp, with_D=False, with_h0=True, tag="no D, h0")


def test_large_dt_and_strong_decay():
    # dt up to ~8 and A down to -16: the decay mask spans many orders of magnitude, and within
    # a 32-token block the decay can pass 2^100, where the output kernel stops factorizing the
    # block's decay and takes each entry's own (both forms occur across the heads here)
    inp = workloads.make_custom_prefill(15, batch=1, seqlen=512, nheads=4, headdim=64, dstate=128, ngroups=1,
                                        chunk=256)
    inp["dt"] = (inp["dt"] * 30).astype(np.float32)
    _check_full(inp, tag="large dt")


def test_no_decay_and_decay_to_zero():
    inp = workloads.make_custom_prefill(16, batch=1, seqlen=384, nheads=2, headdim=32, dstate=64, ngroups=1,
                                        chunk=128, h0_std=0.1)
    inp["A"] = np.zeros_like(inp["A"])
    _check_full(inp, tag="A=0")
    inp["A"] = np.full_like(inp["A"], -1e5)   # every diagonal block past the factorized range
    _check_full(inp, tag="A=-1e5")


def test_strong_decay_with_ragged_tail():
    # the last chunk ends mid-block: past the sequence end dt is 0 while the decay weights of a
    # strongly decaying block overflow, and no inf * 0 may reach the outputs
    inp = workloads.make_custom_prefill(17, batch=2, seqlen=300, nheads=4, headdim=64, dstate=128, ngroups=1,
                                        chunk=128, h0_std=0.1)
    inp["dt"] = (inp["dt"] * 30).astype(np.float32)
    inp["A"][::2] = -1e3
    _check_full(inp, tag="ragged strong decay")


def test_h_final_may_alias_h0():
    import quantized_selective_state_amd as ssdq
    inp = workloads.make_custom_prefill(17, batch=1, seqlen=256, nheads=2, headdim=32, dstate=32, ngroups=1,
                                        chunk=64, h0_std=0.2)
    qx, sx, qB, sB, qC, sC = gpu_quantize_inputs(inp)
    h = to_dev(inp["h0"])
    y, hf = ssdq.chunk_scan(qx, sx, qB, sB, qC, sC, to_dev(inp["dt"]), to_dev(inp["A"]), to_dev(inp["D"]), h,
                            chunk=64, h_final=h)
    c = oracle_codes(inp)
    y_ref, h_ref, _ = oracle.ssd(c)
    assert rel_err(h.cpu().numpy(), h_ref) <= H_TOL
    assert rel_err(y.float().cpu().numpy(), y_ref) <= Y_TOL


def test_stage_intermediates():
    """Acs, chunk states and the states entering each chunk against their oracle definitions."""
    import quantized_selective_state_amd as ssdq
    inp = workloads.make_custom_prefill(18, batch=2, seqlen=600, nheads=4, headdim=64, dstate=128, ngroups=2,
                                        chunk=256, x_dist="outlier_heads", h0_std=0.1)
    qx, sx, qB, sB, qC, sC = gpu_quantize_inputs(inp)
    buf = ssdq.ScanBuffers(qx, sx, qB, sB, qC, sC, to_dev(inp["dt"]), to_dev(inp["A"]), to_dev(inp["D"]),
                           to_dev(inp["h0"]), chunk=256)
    c = oracle_codes(inp)
    views = buf.workspace_views()
    buf.run_stage(0)                       # chunk cumsum + chunk states
    torch.cuda.synchronize()
    acs = views["acs"].cpu().numpy()
    dtc = views["dtc"].cpu().numpy()
    S = views["states"].cpu().numpy().copy()
    buf.run_stage(1)                       # state passing -> carried state as two int8 limbs + row scales
    torch.cuda.synchronize()
    Hprev = carried_state(views["hprev"].cpu().numpy(), views["hscale"].cpu().numpy())
    buf.run_stage(2)                       # chunk output
    torch.cuda.synchronize()
    nc = acs.shape[2]
    _, h_ref, bounds = oracle.ssd(c, chunk=256)
    for b in range(c.batch):
        for h in range(c.H):
            a_ref = oracle.chunk_cumsum(c, b, h, 256)
            valid = np.isfinite(a_ref)
            # fp32 accumulation of up to 256 terms
            assert np.max(np.abs(acs[b, h][valid] - a_ref[valid])) <= 2e-5 * max(1.0, np.max(np.abs(a_ref[valid])))
            # dt in chunk order: the input's values bit for bit, zeros past the sequence end
            d_pad = np.zeros(nc * 256, dtype=np.float32)
            d_pad[:c.L] = inp["dt"][b, :, h]
            assert np.array_equal(dtc[b, h].reshape(-1), d_pad)
            S_ref = oracle.chunk_state(c, b, h, 256)
            # three INT8 limbs (~2^-23 of the chunk max) plus fp32 cumsum/exp of the decay
            assert rel_err(S[b, :, h], S_ref) <= 5e-5
            # the carried state is stored as two int8 limbs (~2^-15 of each row max)
            assert rel_err(Hprev[b, :, h], bounds[b, :, h]) <= 1e-4
    assert nc == 3
    y_ref, _, _ = oracle.ssd(c)
    assert rel_err(buf.y.float().cpu().numpy(), y_ref) <= Y_TOL
    assert rel_err(buf.h_final.cpu().numpy(), h_ref) <= H_TOL


def test_deterministic():
    inp = workloads.make_custom_prefill(19, batch=2, seqlen=512, nheads=8, headdim=64, dstate=128, ngroups=1,
                                        chunk=256, h0_std=0.1)
    _, y1, h1 = gpu_prefill(inp)
    _, y2, h2 = gpu_prefill(inp)
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)


@pytest.mark.parametrize("name", ["mamba2-1.3b-prefill", "mamba2-2.7b-long-prefill", "mamba2-8b-prefill"])
def test_full_workload(name):
    """Whole GPU path at the workload's real size (the launch configuration the benchmark times),
    every (batch, head) sequence against the oracle: codes bit-exact, y and the final state
    within the bars over the whole tensors."""
    import quantized_selective_state_amd as ssdq
    note(f"generating {name}")
    inp = workloads.make_prefill(name)
    note(f"gpu {name}")
    qx, sx, qB, sB, qC, sC = gpu_quantize_inputs(inp)
    h0 = to_dev(inp["h0"])
    y, hf = ssdq.chunk_scan(qx, sx, qB, sB, qC, sC, to_dev(inp["dt"]), to_dev(inp["A"]), to_dev(inp["D"]), h0,
                            chunk=inp["chunk"])
    torch.cuda.synchronize()
    note(f"oracle codes {name}")
    c = oracle_codes(inp)
    del inp
    assert np.array_equal(qx.cpu().numpy(), c.qx), "x codes differ"
    assert np.array_equal(qB.cpu().numpy(), c.qB) and np.array_equal(qC.cpu().numpy(), c.qC)
    del qx, qB, qC
    note(f"oracle {name}: all {c.batch * c.H} sequences")
    compare_full(c, lambda b: y[b].float().cpu().numpy(), lambda b: hf[b].cpu().numpy(), name)


def test_maximum_chunk_count():
    # the longest sequence the scan accepts at chunk 64: 65535 chunks (4,194,240 tokens), one
    # narrow head (three-kernel plan: state passing walks all 65535 chunks in one sequence);
    # one chunk more is refused on the host
    import quantized_selective_state_amd as ssdq
    L = 65535 * 64
    inp = workloads.make_custom_prefill(18, batch=1, seqlen=L, nheads=1, headdim=16, dstate=16, ngroups=1,
                                        chunk=64, h0_std=0.1)
    note(f"maximum chunk count: L={L}")
    _check_full(inp, tag="65535 chunks")
    qx = torch.zeros((1, L + 64, 1, 16), dtype=torch.int8, device=dev())
    qb = torch.zeros((1, L + 64, 1, 16), dtype=torch.int8, device=dev())
    one = torch.ones(1, device=dev())
    with pytest.raises(ssdq.SSDQError) as e:
        ssdq.chunk_scan(qx, one, qb, one, qb, one, torch.zeros((1, L + 64, 1), device=dev()), -one, chunk=64)
    assert e.value.status == ssdq.SSDQ_ERROR_UNSUPPORTED
