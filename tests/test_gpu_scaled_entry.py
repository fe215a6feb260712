"""The scale-layout entry points through the C ABI: ssdq_chunk_scan_scaled and
ssdq_state_update_scaled with layout 0 (per head / per group) and layout 1 (B, C per (group,
state)) run the kernels of ssdq_chunk_scan / ssdq_chunk_scan_per_state and of the decode entry
points, so their outputs are bit-equal to those calls' on the same inputs (both plans of the
scan; the three decode state formats)."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from gpu_util import dev, note, to_dev

pytestmark = pytest.mark.gpu


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _inputs(seed, batch, nheads, per_state):
    shape = workloads.PrefillShape(f"se{seed}", batch, 200, nheads, 32, 64, 2, 64, "outlier_heads", "fixed_bias", 0.2)
    _, inp = workloads.make_calibrated_pair(shape, seed, bc_per_state=per_state, state_spread=1.0 if per_state else 0.0)
    return inp


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("per_state", [False, True])
def test_scan_scaled_equals_the_fixed_layout_calls(fused, per_state):
    import quantized_selective_state_amd as ssdq
    batch, nheads = (-(-_cus() // 16), 16) if fused else (2, 4)
    inp = _inputs(95 + 2 * int(fused) + int(per_state), batch, nheads, per_state)
    assert ssdq.chunk_scan_state_fused(batch, nheads) == fused
    sx, sB, sC = to_dev(inp["x_scale"]), to_dev(inp["B_scale"]), to_dev(inp["C_scale"])
    qx, qB, qC = ssdq.quantize(to_dev(inp["x16"]), sx), ssdq.quantize(to_dev(inp["B16"]), sB), \
        ssdq.quantize(to_dev(inp["C16"]), sC)
    dt, A, D, h0 = to_dev(inp["dt"]), to_dev(inp["A"]), to_dev(inp["D"]), to_dev(inp["h0"])
    y_ref, h_ref = ssdq.chunk_scan(qx, sx, qB, sB, qC, sC, dt, A, D, h0, chunk=inp["chunk"])
    b, L, H, P = qx.shape
    G, N = qB.shape[2], qB.shape[3]
    y = torch.empty_like(y_ref)
    hf = torch.empty_like(h_ref)
    ws = torch.empty(ssdq.chunk_scan_workspace_size(b, L, H, P, N, inp["chunk"]), dtype=torch.uint8, device=dev())
    p = lambda t: ctypes.c_void_p(None if t is None else t.data_ptr())
    layout = ssdq.SCALES_BC_PER_STATE if per_state else 0
    note(f"scaled entry: layout {layout}, fused={fused}")
    st = ssdq.lib.ssdq_chunk_scan_scaled(p(qx), p(sx), p(qB), p(sB), p(qC), p(sC), p(dt), p(A), p(D), p(None), p(h0),
                                         p(y), p(hf), b, L, H, P, N, G, inp["chunk"], layout, p(ws), ws.numel(),
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref) and torch.equal(hf, h_ref)


@pytest.mark.parametrize("fmt", ["f32", "f16", "i8"])
@pytest.mark.parametrize("per_state", [False, True])
def test_state_update_scaled_equals_the_fixed_layout_calls(fmt, per_state):
    import quantized_selective_state_amd as ssdq
    rng = np.random.default_rng(97)
    b, H, P, N, G = 3, 8, 64, 128, 2
    sx = to_dev(rng.uniform(0.01, 0.05, size=H).astype(np.float32))
    sshape = (G, N) if per_state else (G,)
    sB = to_dev(rng.uniform(0.01, 0.05, size=sshape).astype(np.float32))
    sC = to_dev(rng.uniform(0.01, 0.05, size=sshape).astype(np.float32))
    qx = to_dev(rng.integers(-127, 128, size=(b, H, P), dtype=np.int8))
    qB = to_dev(rng.integers(-127, 128, size=(b, G, N), dtype=np.int8))
    qC = to_dev(rng.integers(-127, 128, size=(b, G, N), dtype=np.int8))
    dt = to_dev(rng.uniform(0.01, 0.2, size=(b, H)).astype(np.float32))
    A = to_dev(-rng.uniform(0.5, 4, size=H).astype(np.float32))
    D = to_dev(rng.uniform(0.5, 1.5, size=H).astype(np.float32))
    s0 = rng.normal(0, 0.5, size=(b, H, P, N)).astype(np.float32)
    if fmt == "f32":
        st_a, st_b, sc_a, sc_b = to_dev(s0), to_dev(s0), None, None
    elif fmt == "f16":
        st_a, st_b, sc_a, sc_b = to_dev(s0).half(), to_dev(s0).half(), None, None
    else:
        st_a = to_dev(rng.integers(-127, 128, size=(b, H, P, N), dtype=np.int8))
        st_b = st_a.clone()
        sc_a = to_dev(rng.uniform(0.001, 0.01, size=(b, H, P)).astype(np.float32))
        sc_b = sc_a.clone()
    y_ref = ssdq.state_update(st_a, qx, sx, qB, sB, qC, sC, dt, A, D, state_scale=sc_a)
    y = torch.empty_like(y_ref)
    p = lambda t: ctypes.c_void_p(None if t is None else t.data_ptr())
    fmt_id = {"f32": ssdq.STATE_F32, "f16": ssdq.STATE_F16, "i8": ssdq.STATE_I8}[fmt]
    layout = ssdq.SCALES_BC_PER_STATE if per_state else 0
    st = ssdq.lib.ssdq_state_update_scaled(fmt_id, p(st_b), p(sc_b), p(qx), p(sx), p(qB), p(sB), p(qC), p(sC), p(dt),
                                           p(A), p(D), p(None), p(y), b, H, P, N, G, layout,
                                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref) and torch.equal(st_b, st_a)
    if sc_a is not None:
        assert torch.equal(sc_b, sc_a)
