"""The library's calls under HIP graph capture (torch.cuda.CUDAGraph on ROCm), as a serving loop
or a captured prefill would use them: the captured work is replayed several times, with new
inputs copied in eagerly and the host synchronizing between the replays, and every replay must
equal the same calls made eagerly on the same inputs bit for bit (the same kernels run; no call
of the library records a memset or allocates).

- decode: one step (quantize x, B, C of the token, then the state update on an fp32, a binary16
  or an 8-bit state) captured once and replayed for 6 tokens;
- prefill: ssdq_chunk_scan_noalloc (the static-scratch entry point, for callers that cannot
  allocate, such as code under capture) captured once and replayed on 3 different inputs."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import note, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", ["f32", "f16", "i8"])
def test_decode_step_replayed_equals_eager(fmt):
    import quantized_selective_state_amd as ssdq
    T = 6
    dec = workloads.make_decode(workloads.DecodeShape(f"graph_{fmt}", 8, T, 16, 64, 128, 4, 0.5), seed_index=95)
    sx, sB, sC = to_dev(dec["x_scale"]), to_dev(dec["B_scale"]), to_dev(dec["C_scale"])
    A, D = to_dev(dec["A"]), to_dev(dec["D"])
    x16, B16, C16, dts = to_dev(dec["x16"]), to_dev(dec["B16"]), to_dev(dec["C16"]), to_dev(dec["dt"])

    def fresh_state():
        if fmt == "f32":
            return to_dev(dec["state"]), None
        if fmt == "f16":
            return to_dev(dec["state"]).half(), None
        q0, s0, _ = oracle.requantize_rows_i8(dec["state"].reshape(-1, 128).astype(np.float64))
        return to_dev(q0.reshape(dec["state"].shape)), to_dev(s0.reshape(dec["state"].shape[:3]))

    # static buffers of one step
    xs, Bs, Cs, dts1 = x16[0].clone(), B16[0].clone(), C16[0].clone(), dts[0].clone()
    qx, qB, qC = (torch.empty(t.shape, dtype=torch.int8, device=t.device) for t in (xs, Bs, Cs))
    y = torch.empty(qx.shape, dtype=torch.float16, device=qx.device)

    def one_step(state, scale):
        ssdq.quantize(xs, sx, qx)
        ssdq.quantize(Bs, sB, qB)
        ssdq.quantize(Cs, sC, qC)
        ssdq.state_update(state, qx, sx, qB, sB, qC, sC, dts1, A, D, y=y, state_scale=scale)

    # eager reference
    st_e, sc_e = fresh_state()
    ys_e = []
    for t in range(T):
        xs.copy_(x16[t]), Bs.copy_(B16[t]), Cs.copy_(C16[t]), dts1.copy_(dts[t])
        one_step(st_e, sc_e)
        ys_e.append(y.clone())
    torch.cuda.synchronize()

    # captured: warm up on a side stream as torch asks, then capture one step
    st_g, sc_g = fresh_state()
    warm_state, warm_scale = fresh_state()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        one_step(warm_state, warm_scale)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        one_step(st_g, sc_g)
    torch.cuda.synchronize()
    # capturing does not run the step: restore the state the replays start from
    st0, sc0 = fresh_state()
    st_g.copy_(st0)
    if sc_g is not None:
        sc_g.copy_(sc0)
    torch.cuda.synchronize()
    for t in range(T):
        xs.copy_(x16[t]), Bs.copy_(B16[t]), Cs.copy_(C16[t]), dts1.copy_(dts[t])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ys_e[t]), f"{fmt}: replay {t} differs from the eager step"
    assert torch.equal(st_g, st_e)
    if sc_g is not None:
        assert torch.equal(sc_g, sc_e)
    note(f"graph decode ({fmt} state): {T} replays equal the eager steps")


def test_noalloc_prefill_replayed_equals_eager():
    import quantized_selective_state_amd as ssdq
    draws = [workloads.make_custom_prefill(96 + k, batch=2, seqlen=320, nheads=8, headdim=64, dstate=128,
                                           ngroups=2, chunk=128, x_dist="outlier_heads", h0_std=0.1)
             for k in range(3)]
    d0 = draws[0]
    b, L, H, P, N, G, Q = (d0[k] for k in ("batch", "seqlen", "nheads", "headdim", "dstate", "ngroups", "chunk"))
    sx, sB, sC = to_dev(d0["x_scale"]), to_dev(d0["B_scale"]), to_dev(d0["C_scale"])
    A, D = to_dev(d0["A"]), to_dev(d0["D"])
    # static inputs and outputs (the draws share the model; their data and h0 differ)
    x16, B16, C16 = to_dev(d0["x16"]), to_dev(d0["B16"]), to_dev(d0["C16"])
    dt, h0 = to_dev(d0["dt"]), to_dev(d0["h0"])
    qx = torch.empty(x16.shape, dtype=torch.int8, device=x16.device)
    qB = torch.empty(B16.shape, dtype=torch.int8, device=x16.device)
    qC = torch.empty(C16.shape, dtype=torch.int8, device=x16.device)
    y = torch.empty((b, L, H, P), dtype=torch.float16, device=x16.device)
    hf = torch.empty((b, H, P, N), dtype=torch.float32, device=x16.device)

    def prefill():
        ssdq.quantize(x16, sx, qx)
        ssdq.quantize(B16, sB, qB)
        ssdq.quantize(C16, sC, qC)
        ssdq.chunk_scan_noalloc(qx, sx, qB, sB, qC, sC, dt, A, D, h0, chunk=Q, y=y, h_final=hf)

    def load(d):
        x16.copy_(to_dev(d["x16"])), B16.copy_(to_dev(d["B16"])), C16.copy_(to_dev(d["C16"]))
        dt.copy_(to_dev(d["dt"])), h0.copy_(to_dev(d["h0"]))

    eager = []
    for d in draws:
        load(d)
        prefill()
        torch.cuda.synchronize()
        eager.append((y.clone(), hf.clone()))

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        prefill()   # warm-up (the scratch address is looked up on the first call on a device)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        prefill()
    torch.cuda.synchronize()
    for k, d in enumerate(draws):
        load(d)
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager[k][0]) and torch.equal(hf, eager[k][1]), f"replay {k} differs from the eager call"
    note(f"graph prefill (no-alloc entry point): {len(draws)} replays equal the eager calls")
