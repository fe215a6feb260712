"""GPU check of ssdq_chunk_scan_noalloc, the prefill entry point for callers that cannot allocate:
through the C ABI it must give exactly what ssdq_chunk_scan gives with a workspace (the same
kernels, only the scratch differs), on two calls in a row, the second with a smaller input and
the other plan of the scan, so that the scratch holds the first call's data when the second
starts.  The workspace of the reference call is filled with NaN bytes, so neither path can pass
by reading memory it did not write.  Both are also held to the oracle's bar."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import H_TOL, Y_TOL, gpu_quantize_inputs, note, oracle_codes, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _both(inp):
    import quantized_selective_state_amd as ssdq
    qx, sx, qB, sB, qC, sC = gpu_quantize_inputs(inp)
    dt, A, D, h0 = to_dev(inp["dt"]), to_dev(inp["A"]), to_dev(inp["D"]), to_dev(inp["h0"])
    b, L, H, P, N, Q = (inp[k] for k in ("batch", "seqlen", "nheads", "headdim", "dstate", "chunk"))
    ws = torch.full((ssdq.chunk_scan_workspace_size(b, L, H, P, N, Q),), 0xFF, dtype=torch.uint8, device=qx.device)
    y_ws, h_ws = ssdq.chunk_scan(qx, sx, qB, sB, qC, sC, dt, A, D, h0, chunk=Q, workspace=ws)
    y_na, h_na = ssdq.chunk_scan_noalloc(qx, sx, qB, sB, qC, sC, dt, A, D, h0, chunk=Q)
    torch.cuda.synchronize()
    return (y_ws.float().cpu().numpy(), h_ws.cpu().numpy(), y_na.float().cpu().numpy(), h_na.cpu().numpy(),
            ssdq.chunk_scan_state_fused(b, H))


def test_noalloc_equals_workspace_path_on_two_calls():
    import quantized_selective_state_amd as ssdq
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    big = workloads.make_custom_prefill(81, batch=-(-cus // 64), seqlen=512, nheads=64, headdim=64, dstate=128,
                                        ngroups=2, chunk=128, x_dist="outlier_heads", h0_std=0.1)
    small = workloads.make_custom_prefill(82, batch=1, seqlen=300, nheads=8, headdim=32, dstate=64, ngroups=4,
                                          chunk=64, h0_std=0.2)
    for tag, inp in (("first call, folded plan", big), ("second call, smaller, three-kernel plan", small)):
        need = ssdq.chunk_scan_noalloc_scratch_size(inp["batch"], inp["seqlen"], inp["nheads"], inp["headdim"],
                                                    inp["dstate"], inp["chunk"])
        assert 0 < need <= ssdq.NOALLOC_SCRATCH_BYTES
        y_ws, h_ws, y_na, h_na, fused = _both(inp)
        note(f"no-alloc {tag}: scratch {need} bytes, plan {'folded' if fused else 'three kernels'}")
        assert np.array_equal(y_na, y_ws) and np.array_equal(h_na, h_ws)
        y_ref, h_ref, _ = oracle.ssd(oracle_codes(inp))
        assert rel_err(y_na, y_ref) <= Y_TOL and rel_err(h_na, h_ref) <= H_TOL
    assert ssdq.chunk_scan_state_fused(big["batch"], big["nheads"])
    assert not ssdq.chunk_scan_state_fused(small["batch"], small["nheads"])


def test_noalloc_rejects_shapes_beyond_the_scratch():
    import quantized_selective_state_amd as ssdq
    z8 = lambda *s: torch.zeros(s, dtype=torch.int8, device="cuda")
    z32 = lambda *s: torch.zeros(s, dtype=torch.float32, device="cuda")
    b, L, H, P, N, G, Q = 8, 4096, 128, 64, 128, 8, 256     # the 8B-shaped layer: 256 MiB of carried state
    assert ssdq.chunk_scan_noalloc_scratch_size(b, L, H, P, N, Q) > ssdq.NOALLOC_SCRATCH_BYTES
    with pytest.raises(ssdq.SSDQError) as e:
        ssdq.chunk_scan_noalloc(z8(b, L, H, P), z32(H), z8(b, L, G, N), z32(G), z8(b, L, G, N), z32(G), z32(b, L, H),
                                z32(H), chunk=Q)
    assert e.value.status == ssdq.SSDQ_ERROR_SCRATCH_LIMIT
