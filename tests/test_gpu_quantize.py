"""GPU parity of ssdq_quantize: codes must equal the oracle's bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import dev, note, to_dev

pytestmark = pytest.mark.gpu

ALL_F16 = np.arange(65536, dtype=np.uint16).view(np.float16)
SCALES = [1.0, 0.5, 1.0 / 127.0, 3.0, 0.3, 0.0123, 2.0 ** -20, 0.8160377, 37.5]


@pytest.mark.parametrize("inner", [8, 1])   # vector path (8 per thread) and scalar path
def test_every_f16_value_every_scale(inner):
    import quantized_selective_state_amd as ssdq
    scales = np.array(SCALES, dtype=np.float32)
    # (rows, nscale, inner): every scale sees all 65536 fp16 inputs
    x = np.ascontiguousarray(np.repeat(ALL_F16.reshape(65536 // inner, 1, inner), len(SCALES), axis=1))
    note(f"quantize exhaustive inner={inner} shape={x.shape}")
    got = ssdq.quantize(to_dev(x), to_dev(scales)).cpu().numpy()
    ref = oracle.quantize(x, scales)
    bad = np.count_nonzero(got != ref)
    assert bad == 0, f"{bad} code mismatches"


@pytest.mark.parametrize("name", ["tiny", "mamba2-1.3b-prefill"])
def test_workload_tensors(name):
    import quantized_selective_state_amd as ssdq
    inp = workloads.make_prefill(name)
    for key, skey in (("x16", "x_scale"), ("B16", "B_scale"), ("C16", "C_scale")):
        note(f"quantize {name} {key} {inp[key].shape}")
        got = ssdq.quantize(to_dev(inp[key]), to_dev(inp[skey])).cpu().numpy()
        ref = oracle.quantize(inp[key], inp[skey])
        assert np.array_equal(got, ref), f"{key}: {np.count_nonzero(got != ref)} mismatches"
        if key == "x16":
            # outlier heads saturate nowhere in calibration range, but the test draw can exceed it
            assert np.abs(got.astype(np.int32)).max() <= 127


@pytest.mark.parametrize("shape", [(37, 3, 5), (1, 1, 1), (5, 2, 12), (3, 4, 16)])
def test_ragged_shapes(shape):
    import quantized_selective_state_amd as ssdq
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(shape) * 30).astype(np.float16)
    s = rng.uniform(0.05, 1.0, size=shape[1]).astype(np.float32)
    got = ssdq.quantize(to_dev(x), to_dev(s)).cpu().numpy()
    assert np.array_equal(got, oracle.quantize(x, s))


def test_empty_rows_is_a_noop():
    import quantized_selective_state_amd as ssdq
    x = torch.empty((0, 4, 16), dtype=torch.float16, device=dev())
    out = ssdq.quantize(x, torch.ones(4, device=dev()))
    assert out.shape == (0, 4, 16)


@pytest.mark.parametrize("name", ["tiny", "mamba2-1.3b-prefill"])
def test_batch_equals_the_oracle(name):
    """x, B, C of a workload in one batched call, plus a ragged tensor (its own launch) and an
    empty one: every code equals the oracle's."""
    import quantized_selective_state_amd as ssdq
    inp = workloads.make_prefill(name)
    rng = np.random.default_rng(11)
    rag = (rng.standard_normal((37, 3, 5)) * 30).astype(np.float16)
    rag_s = rng.uniform(0.05, 1.0, size=3).astype(np.float32)
    pairs = [(inp["x16"], inp["x_scale"]), (inp["B16"], inp["B_scale"]), (inp["C16"], inp["C_scale"]),
             (rag, rag_s), (np.zeros((0, 2, 16), np.float16), np.ones(2, np.float32))]
    note(f"quantize batch {name}: {[p[0].shape for p in pairs]}")
    got = ssdq.quantize_batch([(to_dev(x), to_dev(s)) for x, s in pairs])
    for (x, s), g in zip(pairs, got):
        ref = oracle.quantize(x, s)
        g = g.cpu().numpy()
        assert g.shape == ref.shape
        assert np.array_equal(g, ref), f"{x.shape}: {np.count_nonzero(g != ref)} mismatches"


def test_batch_into_given_outputs_twice():
    """Outputs passed in are written in place; a second run with new inputs overwrites them."""
    import quantized_selective_state_amd as ssdq
    rng = np.random.default_rng(12)
    shapes = [(64, 4, 32), (64, 1, 128), (64, 1, 128)]
    outs = [torch.full(s, 99, dtype=torch.int8, device=dev()) for s in shapes]
    for rep in range(2):
        xs = [(rng.standard_normal(s) * (20 + 10 * rep)).astype(np.float16) for s in shapes]
        ss = [rng.uniform(0.05, 1.0, size=s[1]).astype(np.float32) for s in shapes]
        batch = ssdq.QuantizeBatch([ssdq.QuantizeCall(to_dev(x), to_dev(s), o) for x, s, o in zip(xs, ss, outs)])
        got = batch.run()
        for x, s, g, o in zip(xs, ss, got, outs):
            assert g.data_ptr() == o.data_ptr()
            assert np.array_equal(g.cpu().numpy(), oracle.quantize(x, s))
