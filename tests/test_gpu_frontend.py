"""GPU parity of ssdq_frontend: depthwise causal conv1d + bias + SiLU, binary16, static INT8
codes, and dt = softplus(dt_raw + dt_bias), against the oracle.

The kernel forms the SiLU value in fp32 and rounds it to binary16; the oracle in double.  They
can part only where the exact value lies within the kernel's fp32 error of a midpoint between
two binary16 neighbours; everywhere else the binary16 value, hence the code (the quantizer is
bit-exact), must be the oracle's.  The band is derived per element from the kernel's arithmetic
(unit roundoff e = 2^-24; v the convolution plus bias, S = |bias| + sum_k |w_k x_k|):
  - the four fused multiply-adds of the convolution: |v_gpu - v| <= 4 e S;
  - exp(-v) as exp2 of a rounded product (the ulp-accurate hardware exp2): relative
    (|v| + 1) 2e; 1 + exp(-v): e; the hardware reciprocal: 2e; the product v / (1 + exp(-v)): e;
  - SiLU's slope is below 1.1, so |silu_gpu - silu(v)| <= 1.1 (4 e S) + |silu(v)| ((|v| + 1) 2e + 4e).
Near a midpoint (within twice that bound) the code of either neighbour is accepted.  dt is
compared to a relative 1e-6 (a few fp32 roundings)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import dev, note, to_dev

pytestmark = pytest.mark.gpu

EPS = 2.0 ** -24
SAFETY = 2.0


def _silu_error_bound(fe, pre: np.ndarray, act: np.ndarray) -> np.ndarray:
    """Per-element bound on the kernel's fp32 SiLU error (see the module docstring)."""
    x = fe["xbc16"].astype(np.float64)                # (b, L, C)
    w = fe["conv_w"].astype(np.float64)               # (C, 4): tap k meets token t - 3 + k
    S = np.zeros_like(x) if fe["conv_b"] is None else np.broadcast_to(np.abs(fe["conv_b"].astype(np.float64)),
                                                                        x.shape).copy()
    L = x.shape[1]
    for k in range(4):
        lag = 3 - k
        S[:, lag:] += np.abs(w[:, k]) * np.abs(x[:, :L - lag])
    return SAFETY * (1.1 * 4 * EPS * S + np.abs(act) * ((np.abs(pre) + 1) * 2 * EPS + 4 * EPS))


def _gpu(fe):
    import quantized_selective_state_amd as ssdq
    H, P, G, N = fe["nheads"], fe["headdim"], fe["ngroups"], fe["dstate"]
    x, B, C, dt = ssdq.frontend(to_dev(fe["xbc16"]), to_dev(fe["conv_w"]), to_dev(fe["conv_b"]),
                                to_dev(fe["x_scale"]), to_dev(fe["B_scale"]), to_dev(fe["C_scale"]),
                                to_dev(fe["dt_raw"]), to_dev(fe["dt_bias"]), H, P, G, N)
    torch.cuda.synchronize()
    return x.cpu().numpy(), B.cpu().numpy(), C.cpu().numpy(), dt.cpu().numpy()


def _check(fe, tag, got=None):
    H, P, G, N = fe["nheads"], fe["headdim"], fe["ngroups"], fe["dstate"]
    b, L = fe["batch"], fe["seqlen"]
    qx, qB, qC, dt = _gpu(fe) if got is None else got
    ref = oracle.frontend(fe["xbc16"], fe["conv_w"], fe["conv_b"], fe["x_scale"], fe["B_scale"], fe["C_scale"],
                          H, P, G, N)
    act, a16 = ref["act"], ref["act16"]
    bound = _silu_error_bound(fe, ref["pre"], act)
    up = act >= a16.astype(np.float64)
    other = np.where(up, np.nextafter(a16, np.float16(np.inf)), np.nextafter(a16, np.float16(-np.inf)))
    spacing = np.abs(other.astype(np.float64) - a16.astype(np.float64))
    mid = (other.astype(np.float64) + a16.astype(np.float64)) / 2
    near = np.abs(act - mid) <= bound
    normal = np.abs(a16.astype(np.float64)) >= 2.0 ** -14      # the band in spacings, normal binary16 values
    widest = float(np.max(bound[normal] / spacing[normal])) if normal.any() else 0.0
    hp, gn = H * P, G * N
    parts = [("x", qx, ref["qx"], slice(0, hp), (H, P), fe["x_scale"]),
             ("B", qB, ref["qB"], slice(hp, hp + gn), (G, N), fe["B_scale"]),
             ("C", qC, ref["qC"], slice(hp + gn, hp + 2 * gn), (G, N), fe["C_scale"])]
    n_near = n_diff = 0
    for name, got, want, sl, shp, scale in parts:
        alt = oracle.quantize(other[..., sl].reshape(b, L, *shp), scale)
        nr = near[..., sl].reshape(b, L, *shp)
        diff = got != want
        assert not np.any(diff & ~nr), f"{name}: {int(np.sum(diff & ~nr))} codes differ away from a midpoint"
        assert np.all(got[diff] == alt[diff]), f"{name}: a code near a midpoint is neither neighbour's"
        n_near += int(nr.sum())
        n_diff += int(diff.sum())
    dref = oracle.softplus_dt(fe["dt_raw"], fe["dt_bias"])
    e_dt = float(np.max(np.abs(dt - dref) / np.abs(dref)))
    note(f"{tag}: {qx.size + qB.size + qC.size} codes, {n_near} within the derived band of a binary16 midpoint "
         f"(at most {widest:.2e} of a spacing for normal values), {n_diff} differ; dt rel {e_dt:.2e}")
    assert e_dt <= 1e-6


def test_tiny():
    _check(workloads.make_frontend("tiny"), "tiny")


def test_ragged_tokens_two_groups_no_bias():
    shape = workloads.PrefillShape("fe_ragged", 2, 77, 6, 32, 64, 2, 64, "normal", "fixed_bias", 0.0)
    fe = workloads.make_frontend(shape, seed_index=31)
    fe["conv_b"] = None
    fe["dt_bias"] = None
    _check(fe, "ragged L=77, G=2, no bias")


def test_prefill_workload_full():
    fe = workloads.make_frontend("mamba2-1.3b-prefill")
    _check(fe, "mamba2-1.3b-prefill")


def test_empty_sequence_is_a_noop():
    import quantized_selective_state_amd as ssdq
    fe = workloads.make_frontend("tiny")
    H, P, G, N = fe["nheads"], fe["headdim"], fe["ngroups"], fe["dstate"]
    z = lambda *s, dt=torch.int8: torch.zeros(s, dtype=dt, device=dev())
    out = (z(1, 0, H, P), z(1, 0, G, N), z(1, 0, G, N), z(1, 0, H, dt=torch.float32))
    ssdq.frontend(to_dev(fe["xbc16"][:, :0]), to_dev(fe["conv_w"]), None, to_dev(fe["x_scale"]),
                  to_dev(fe["B_scale"]), to_dev(fe["C_scale"]), to_dev(fe["dt_raw"][:, :0]), None, H, P, G, N, out=out)
    torch.cuda.synchronize()


def test_decode_steps_equal_the_prefill_front_end():
    """Token-by-token steps from a zero conv state give every token the codes and dt of the
    prefill front end over the whole sequence (checked against the oracle, and bit for bit
    against the GPU's own prefill pass, which does the same arithmetic), and leave the last
    three tokens' inputs in the state."""
    import quantized_selective_state_amd as ssdq
    shape = workloads.PrefillShape("fe_steps", 3, 12, 4, 32, 64, 2, 64, "normal", "fixed_bias", 0.0)
    fe = workloads.make_frontend(shape, seed_index=33)
    H, P, G, N = fe["nheads"], fe["headdim"], fe["ngroups"], fe["dstate"]
    b, L = fe["batch"], fe["seqlen"]
    xbc = to_dev(fe["xbc16"])
    w, cb = to_dev(fe["conv_w"]), to_dev(fe["conv_b"])
    sx, sB, sC = to_dev(fe["x_scale"]), to_dev(fe["B_scale"]), to_dev(fe["C_scale"])
    raw, dtb = to_dev(fe["dt_raw"]), to_dev(fe["dt_bias"])
    state = torch.zeros((b, 3, xbc.shape[2]), dtype=torch.float16, device=dev())
    steps = [ssdq.frontend_step(state, xbc[:, t].contiguous(), w, cb, sx, sB, sC, raw[:, t].contiguous(), dtb,
                                H, P, G, N) for t in range(L)]
    torch.cuda.synchronize()
    got = tuple(torch.stack([st[k] for st in steps], dim=1).cpu().numpy() for k in range(4))
    _check(fe, "decode steps", got=got)
    pre = _gpu(fe)
    for k in range(4):
        assert np.array_equal(got[k], pre[k])
    assert np.array_equal(state.cpu().numpy(), fe["xbc16"][:, L - 3:])


@pytest.mark.parametrize("name", ["tiny", "ragged"])
def test_front_end_then_scan_matches_the_oracle(name):
    """The prefill step with the front end in place of the quantizer: the front end's codes and
    dt go straight into the chunked scan; y and the final state against the oracle's front end
    followed by the fp64 sequential recurrence."""
    import quantized_selective_state_amd as ssdq
    from gpu_util import Y_TOL
    if name == "tiny":
        fe = workloads.make_frontend("tiny")
    else:
        shape = workloads.PrefillShape("fe_scan", 2, 77, 6, 32, 64, 2, 64, "normal", "fixed_bias", 0.0)
        fe = workloads.make_frontend(shape, seed_index=34)
    H, P, G, N = fe["nheads"], fe["headdim"], fe["ngroups"], fe["dstate"]
    sx, sB, sC = to_dev(fe["x_scale"]), to_dev(fe["B_scale"]), to_dev(fe["C_scale"])
    qx, qB, qC, dt = ssdq.frontend(to_dev(fe["xbc16"]), to_dev(fe["conv_w"]), to_dev(fe["conv_b"]), sx, sB, sC,
                                   to_dev(fe["dt_raw"]), to_dev(fe["dt_bias"]), H, P, G, N)
    y, hf = ssdq.chunk_scan(qx, sx, qB, sB, qC, sC, dt, to_dev(fe["A"]), to_dev(fe["D"]), None, chunk=fe["chunk"])
    torch.cuda.synchronize()
    ref = oracle.frontend(fe["xbc16"], fe["conv_w"], fe["conv_b"], fe["x_scale"], fe["B_scale"], fe["C_scale"],
                          H, P, G, N)
    dt_ref = oracle.softplus_dt(fe["dt_raw"], fe["dt_bias"]).astype(np.float32)
    codes = oracle.Codes(ref["qx"], fe["x_scale"], ref["qB"], fe["B_scale"], ref["qC"], fe["C_scale"], dt_ref,
                         fe["A"], fe["D"])
    y_ref, h_ref, _ = oracle.ssd(codes)
    ey = np.max(np.abs(y.float().cpu().numpy() - y_ref)) / np.max(np.abs(y_ref))
    eh = np.max(np.abs(hf.cpu().numpy() - h_ref)) / np.max(np.abs(h_ref))
    note(f"front end + scan ({name}): y {ey:.2e}, h {eh:.2e}")
    assert ey <= Y_TOL and eh <= 1e-4
