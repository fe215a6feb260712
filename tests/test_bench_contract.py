"""Host-side parts of bench.py that need no GPU: the one-GPU guard, the algorithmic byte
counts the roofline divides by, and the lookup of counter-measured traffic by source digest."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_of_the_prefill_step():
    # mamba2-1.3b-prefill: b 4, L 2048, H 64, P 64, N 128, G 1, Q 256 -> 8192 tokens, 8 chunks
    kb = bench.kernel_bytes(4, 2048, 64, 64, 128, 1, 256)
    tok = 4 * 2048
    x = tok * 64 * 64                      # int8 codes
    bc = tok * 1 * 128                     # int8 codes of B (and of C)
    dt = tok * 64 * 4
    acs = 4 * 64 * 8 * 256 * 4
    limbs = 4 * 8 * 64 * 64 * 128 * 2 + 4 * 8 * 64 * 64 * 4   # two int8 planes + fp32 row scales
    hfin = 4 * 64 * 64 * 128 * 4
    y = tok * 64 * 64 * 2                  # fp16 output
    assert kb["quantize"] == 3 * (x + 2 * bc)                       # fp16 in, int8 out
    dtc = acs                              # dt in chunk order: written by the state stage, read by the output
    assert kb["state_scan"] == x + bc + dt + acs + dtc + limbs + hfin
    assert kb["chunk_output"] == x + 2 * bc + dtc + acs + limbs + y
    # the per-token figures quoted in the design notes
    assert kb["quantize"] / tok == 13056
    assert kb["state_scan"] / tok == 10176
    assert kb["chunk_output"] / tok == 17216


def test_scan_ops_count_causal_pairs_once():
    ops = bench.scan_ops(1, 4, 1, 1, 1, 1, 2)   # two chunks of 2 tokens: 3 causal pairs each
    assert ops["cb_int8"] == 2 * 1 * 1 * (3 + 3) * 1
    assert ops["chunk_state"] == 2 * 1 * 4 * 1 * 1 * 1


def test_traffic_is_reported_only_for_the_current_source(tmp_path, monkeypatch):
    digest = bench.source_digest("chunk_output")
    table = tmp_path / "hbm_traffic_mamba2-8b-prefill.md"
    table.write_text(
        "| kernel | source digest | dispatches | a | b | c | d | e | traffic bytes |\n"
        "|---|---|---|---|---|---|---|---|---|\n"
        f"| chunk_output | {digest} | 5 | 1 | 2 | 3 | 4 | 5 | 123456 |\n"
        "| state_scan | 0000000000000000 | 5 | 1 | 2 | 3 | 4 | 5 | 999 |\n")
    monkeypatch.setattr(bench, "TRAFFIC_DIR", str(tmp_path))
    assert bench.measured_traffic("chunk_output", "mamba2-8b-prefill") == 123456
    assert bench.measured_traffic("state_scan", "mamba2-8b-prefill") is None      # stale digest
    assert bench.measured_traffic("quantize", "mamba2-8b-prefill") is None        # no row
    assert bench.measured_traffic("chunk_output", "mamba2-1.3b-prefill") is None  # no table


@pytest.mark.parametrize("shape,quant,scan", [((64, 64, 128, 1, 256), 13056, 21248),
                                              ((80, 64, 128, 1, 256), 16128, 26496),
                                              ((128, 64, 128, 8, 256), 30720, 44032)])
def test_specified_bytes_per_token(shape, quant, scan):
    """The per-token traffic the roofline is priced by, for the three prefill shapes (H, P, N,
    G, Q): x, B, C int8 in, dt and Acs fp32, the fp32 state entering each chunk, y fp16 out."""
    u = bench.specified_bytes_per_token(*shape)
    assert u["quantize"] == quant and u["chunk_scan"] == scan


def test_headline_is_the_largest_prefill_workload():
    import workloads
    sizes = {n: workloads.WORKLOADS[n].tokens * workloads.WORKLOADS[n].nheads for n in bench.PREFILL_WORKLOADS}
    assert "tiny" in bench.PREFILL_WORKLOADS and "tiny" in bench.LATENCY_ONLY
    assert bench.HEADLINE == max(sizes, key=sizes.get) == "mamba2-8b-prefill"
    assert bench.parse([]).workload is None          # default: every prefill workload


def test_digest_follows_the_kernel_source():
    assert len(bench.source_digest("quantize")) == 16
    assert bench.source_digest("state_scan") == bench.source_digest("chunk_state")   # one file
    assert bench.source_digest("quantize") != bench.source_digest("chunk_output")


def test_digest_ignores_comments_only():
    code = "int a; // note\n/* block\n comment */\nint b;\n\n"
    assert bench._code_only(code) == "int a;\nint b;"
    assert bench._code_only(code.replace("note", "another note")) == bench._code_only(code)
    assert bench._code_only(code.replace("int b", "int c")) != bench._code_only(code)


@pytest.mark.parametrize("kernel", sorted(bench.KERNEL_SOURCE))
def test_every_kernel_maps_to_an_existing_source(kernel):
    path = os.path.join(ROOT, "quantized_selective_state_amd", "csrc", bench.KERNEL_SOURCE[kernel])
    assert os.path.exists(path)
