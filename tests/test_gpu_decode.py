"""GPU parity of ssdq_state_update (decode) against the fp64 oracle, every step.

The decode oracle is the same recurrence run over the decode tokens with the
decode state as h0; step t's GPU output y_t is compared with the oracle's y_t.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import H_TOL, Y_TOL, compare_full, dev, note, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _gpu_decode(dec, with_D=True):
    """Quantize every step's x, B, C and run `steps` state updates; returns (y (T,b,H,P), state, codes)."""
    import quantized_selective_state_amd as ssdq
    sx, sB, sC = to_dev(dec["x_scale"]), to_dev(dec["B_scale"]), to_dev(dec["C_scale"])
    qx = ssdq.quantize(to_dev(dec["x16"]), sx)
    qB = ssdq.quantize(to_dev(dec["B16"]), sB)
    qC = ssdq.quantize(to_dev(dec["C16"]), sC)
    dt, A = to_dev(dec["dt"]), to_dev(dec["A"])
    D = to_dev(dec["D"]) if with_D else None
    state = to_dev(dec["state"])
    T = dec["x16"].shape[0]
    ys = torch.empty((T,) + tuple(qx.shape[1:]), dtype=torch.float16, device=dev())
    for t in range(T):
        ssdq.state_update(state, qx[t], sx, qB[t], sB, qC[t], sC, dt[t], A, D, y=ys[t])
    torch.cuda.synchronize()
    return ys.float().cpu().numpy(), state.cpu().numpy(), qx.cpu().numpy()


def _small_decode(seed, b, H, P, N, G, T):
    shape = workloads.DecodeShape(f"dec{seed}", b, T, H, P, N, G, 0.5)
    return workloads.make_decode(shape, seed_index=seed)


@pytest.mark.parametrize("N,G", [(128, 4), (64, 2), (128, 1)])
def test_small_decode_every_step(N, G):
    dec = _small_decode(30 + N, b=4, H=8, P=64, N=N, G=G, T=16)
    y, st, qx = _gpu_decode(dec)
    c = oracle.decode_as_prefill(dec)
    assert np.array_equal(np.swapaxes(qx, 0, 1), c.qx)
    y_ref, h_ref, _ = oracle.ssd(c)                    # y_ref (b, T, H, P)
    y_ref = np.swapaxes(y_ref, 0, 1)
    ey, eh = rel_err(y, y_ref), rel_err(st, h_ref)
    note(f"decode N={N} G={G}: y_err={ey:.3e} h_err={eh:.3e}")
    assert ey <= Y_TOL and eh <= H_TOL
    # every single step meets the y bound on its own
    for t in range(y.shape[0]):
        assert rel_err(y[t], y_ref[t]) <= Y_TOL


def test_decode_headdim_below_64_and_no_D():
    dec = _small_decode(40, b=3, H=4, P=24, N=128, G=2, T=5)
    y, st, _ = _gpu_decode(dec, with_D=False)
    c = oracle.decode_as_prefill(dec)
    c.D = None
    y_ref, h_ref, _ = oracle.ssd(c)
    assert rel_err(y, np.swapaxes(y_ref, 0, 1)) <= Y_TOL
    assert rel_err(st, h_ref) <= H_TOL


def test_decode_matches_prefill():
    """The same tokens through ssdq_state_update one at a time and through ssdq_chunk_scan."""
    import quantized_selective_state_amd as ssdq
    dec = _small_decode(41, b=2, H=8, P=64, N=128, G=2, T=128)
    y_dec, st_dec, _ = _gpu_decode(dec)
    c = oracle.decode_as_prefill(dec)                  # prefill layout: (b, T, ...)
    y, hf = ssdq.chunk_scan(to_dev(c.qx), to_dev(c.sx), to_dev(c.qB), to_dev(c.sB), to_dev(c.qC), to_dev(c.sC),
                            to_dev(c.dt), to_dev(c.A), to_dev(c.D), to_dev(c.h0), chunk=64)
    y_pre = np.swapaxes(y.float().cpu().numpy(), 0, 1)
    y_ref, h_ref, _ = oracle.ssd(c)
    y_ref = np.swapaxes(y_ref, 0, 1)
    assert rel_err(y_pre, y_ref) <= Y_TOL and rel_err(y_dec, y_ref) <= Y_TOL
    assert rel_err(hf.cpu().numpy(), h_ref) <= H_TOL and rel_err(st_dec, h_ref) <= H_TOL
    assert rel_err(y_dec, y_pre) <= 2 * Y_TOL


def test_full_decode_workload():
    """batch 256, 128 heads, 8 groups, 128 steps on the 1 GiB state: every step's y and the final
    state of every (batch, head) sequence against the oracle."""
    note("generating decode workload")
    dec = workloads.make_decode("mamba2-8b-decode")
    note("gpu decode 128 steps")
    y, st, qx = _gpu_decode(dec)                       # y (T, b, H, P)
    assert np.array_equal(qx, oracle.quantize(dec["x16"], dec["x_scale"]))
    c = oracle.decode_as_prefill(dec)
    del dec
    note(f"oracle decode: all {c.batch * c.H} sequences")
    compare_full(c, lambda b: y[:, b], lambda b: st[b], "decode full")
