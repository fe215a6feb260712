"""GPU parity over seeded random shapes inside the supported envelope (headdim and dstate
multiples of 16 up to 64 and 128, any ngroups dividing nheads, chunk 64/128/256, any seqlen,
with or without D and h0, per-group or per-(group, state) B/C scales, with or without the output
correction), against the oracle at the scan's bars: y within 2e-3 and h_final within 1e-4 of the
largest reference value, codes bit-exact.  A first set has few sequences (the three-kernel plan),
a second one CUs to 4 x CUs sequences (the folded state kernel in blocks of eight or four waves)
with x scales per (head, channel) as another random axis.  The shapes are drawn by a fixed
generator, so the cases are the same on every run."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import H_TOL, Y_TOL, note, rel_err, to_dev

pytestmark = pytest.mark.gpu

CASES = 16


def _case(k):
    rng = np.random.default_rng(4000 + k)
    G = int(rng.choice([1, 2, 4]))
    H = G * int(rng.integers(1, 4))
    P = int(rng.choice([16, 32, 48, 64]))
    N = 16 * int(rng.integers(1, 9))
    Q = int(rng.choice([64, 128, 256]))
    L = int(rng.integers(1, 3 * Q + 50))
    b = int(rng.integers(1, 4))
    return dict(b=b, L=L, H=H, P=P, N=N, G=G, Q=Q, h0=bool(rng.integers(0, 2)), D=bool(rng.integers(0, 2)),
                per_state=bool(rng.integers(0, 2)), corr=bool(rng.integers(0, 2)),
                x_dist=str(rng.choice(["normal", "outlier_heads", "lognormal_heads"])))


@pytest.mark.parametrize("k", range(CASES))
def test_random_shape(k):
    import quantized_selective_state_amd as ssdq
    c = _case(k)
    tag = ", ".join(f"{n}={v}" for n, v in c.items())
    note(f"case {k}: {tag}")
    shape = workloads.PrefillShape(f"rand{k}", c["b"], c["L"], c["H"], c["P"], c["N"], c["G"], c["Q"],
                                   c["x_dist"], "fixed_bias", 0.1 if c["h0"] else 0.0)
    _, inp = workloads.make_calibrated_pair(shape, 700 + k, bc_per_state=c["per_state"],
                                            state_spread=1.0 if c["per_state"] else 0.0)
    mu = np.random.default_rng(800 + k).normal(0, 0.05, size=(c["H"], c["P"])).astype(np.float32) if c["corr"] else None
    sx, sB, sC = to_dev(inp["x_scale"]), to_dev(inp["B_scale"]), to_dev(inp["C_scale"])
    qx, qB, qC = ssdq.quantize(to_dev(inp["x16"]), sx), ssdq.quantize(to_dev(inp["B16"]), sB), \
        ssdq.quantize(to_dev(inp["C16"]), sC)
    D = to_dev(inp["D"]) if c["D"] else None
    h0 = to_dev(inp["h0"]) if c["h0"] else None
    y, hf = ssdq.chunk_scan(qx, sx, qB, sB, qC, sC, to_dev(inp["dt"]), to_dev(inp["A"]), D, h0, chunk=c["Q"],
                            y_corr=None if mu is None else to_dev(mu))
    torch.cuda.synchronize()
    codes = oracle.codes_from_inputs(inp)
    assert np.array_equal(qx.cpu().numpy(), codes.qx) and np.array_equal(qB.cpu().numpy(), codes.qB) \
        and np.array_equal(qC.cpu().numpy(), codes.qC)
    if not c["D"]:
        codes.D = None
    if not c["h0"]:
        codes.h0 = None
    codes.y_corr = mu
    y_ref, h_ref, _ = oracle.ssd(codes)
    y, hf = y.float().cpu().numpy(), hf.cpu().numpy()
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(hf))
    ey, eh = rel_err(y, y_ref), rel_err(hf, h_ref)
    note(f"case {k}: y_err={ey:.3e} h_err={eh:.3e}")
    assert ey <= Y_TOL and eh <= H_TOL


FOLDED_CASES = 8


def _folded_case(k, cus):
    """A shape with at least as many (batch, head) sequences as CUs (the folded state kernel, in
    blocks of eight or four waves), with x scales per (head, channel) as another random axis."""
    rng = np.random.default_rng(5000 + k)
    H = int(rng.choice([32, 64, 80, 128]))
    G = int(rng.choice([g for g in (1, 2, 4, 8) if H % g == 0]))
    target = int(rng.integers(cus, 4 * cus + 1))
    b = -(-target // H)
    P = int(rng.choice([16, 32, 48, 64]))
    N = 16 * int(rng.integers(1, 9))
    Q = int(rng.choice([64, 128, 256]))
    L = int(rng.integers(1, 2 * Q + 50))
    return dict(b=b, L=L, H=H, P=P, N=N, G=G, Q=Q, h0=bool(rng.integers(0, 2)), D=bool(rng.integers(0, 2)),
                per_state=bool(rng.integers(0, 2)), x_clusters=int(rng.choice([0, 2, P // 8])),
                corr=bool(rng.integers(0, 2)), x_dist=str(rng.choice(["normal", "outlier_heads", "lognormal_heads"])))


@pytest.mark.parametrize("k", range(FOLDED_CASES))
def test_random_folded_shape(k):
    import quantized_selective_state_amd as ssdq
    c = _folded_case(k, torch.cuda.get_device_properties(0).multi_processor_count)
    layout = (ssdq.SCALES_BC_PER_STATE if c["per_state"] else 0) | (ssdq.SCALES_X_PER_CHANNEL if c["x_clusters"] else 0)
    plan = ssdq.chunk_scan_plan(c["b"], c["H"], layout)
    assert plan in (4, 8)
    tag = ", ".join(f"{n}={v}" for n, v in c.items())
    note(f"folded case {k} (blocks of {plan} waves): {tag}")
    shape = workloads.PrefillShape(f"randf{k}", c["b"], c["L"], c["H"], c["P"], c["N"], c["G"], c["Q"],
                                   c["x_dist"], "fixed_bias", 0.1 if c["h0"] else 0.0)
    _, inp = workloads.make_calibrated_pair(shape, 900 + k, bc_per_state=c["per_state"],
                                            state_spread=1.0 if c["per_state"] else 0.0,
                                            channel_spread=1.0 if c["x_clusters"] else 0.0,
                                            x_clusters=c["x_clusters"] or None)
    mu = np.random.default_rng(950 + k).normal(0, 0.05, size=(c["H"], c["P"])).astype(np.float32) if c["corr"] else None
    sx, sB, sC = to_dev(inp["x_scale"]), to_dev(inp["B_scale"]), to_dev(inp["C_scale"])
    qx, qB, qC = ssdq.quantize(to_dev(inp["x16"]), sx), ssdq.quantize(to_dev(inp["B16"]), sB), \
        ssdq.quantize(to_dev(inp["C16"]), sC)
    D = to_dev(inp["D"]) if c["D"] else None
    h0 = to_dev(inp["h0"]) if c["h0"] else None
    y, hf = ssdq.chunk_scan(qx, sx, qB, sB, qC, sC, to_dev(inp["dt"]), to_dev(inp["A"]), D, h0, chunk=c["Q"],
                            y_corr=None if mu is None else to_dev(mu))
    torch.cuda.synchronize()
    codes = oracle.codes_from_inputs(inp)
    assert np.array_equal(qx.cpu().numpy(), codes.qx) and np.array_equal(qB.cpu().numpy(), codes.qB) \
        and np.array_equal(qC.cpu().numpy(), codes.qC)
    if not c["D"]:
        codes.D = None
    if not c["h0"]:
        codes.h0 = None
    codes.y_corr = mu
    y_ref, h_ref, _ = oracle.ssd(codes)
    y, hf = y.float().cpu().numpy(), hf.cpu().numpy()
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(hf))
    ey, eh = rel_err(y, y_ref), rel_err(hf, h_ref)
    note(f"folded case {k}: y_err={ey:.3e} h_err={eh:.3e}")
    assert ey <= Y_TOL and eh <= H_TOL
