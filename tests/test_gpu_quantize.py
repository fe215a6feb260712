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
