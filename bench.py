"""Benchmark of the INT8-input Mamba-2 SSD scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME ...]

A step is one pass of the prefill hot path: static INT8 quantize of x, B and C (one batched
launch), then the chunked scan (chunk cumsum, chunk state, state passing, chunk output; with a
(batch, head) sequence per CU the first kernel also carries the state across chunks).  The
headline line is the Mamba-2 8B-shaped layer (batch 8, L 4096, 128 heads x 64, d_state 128,
8 groups, chunk 256: 32,768 tokens per step), the largest prefill configuration; the 1.3B-shaped
layer (batch 4, L 2048, 64 heads, 1 group) and the 2.7B-shaped long sequence (batch 1,
L 16384, 80 heads, nonzero initial state) are measured in the same run under `workloads`.
Inputs are seeded synthetic fp16 activations resident in HBM before timing starts.
Per-kernel times come from a pass with events around every kernel; the timed steps carry
events only around the dominant kernel and the region.  The front end (conv1d + SiLU +
quantize) is measured on the headline shape; the decode update on the 8B-shaped decode
workload (batch 256, 128 heads, 8 groups, 128 steps, 1 GiB fp32 state), one launch per step,
and on the binary16 and 8-bit cached states.  The CPU oracle is timed on the host cores on the
headline workload (and on one thread on a sample of the 1.3B-shaped one).  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_OPS = 5.0e15         # MI355X dense INT8 MFMA
METRIC = "SSD scan tokens/s + % INT8 MFMA peak (prefill); decode HBM GB/s"


# HBM bytes per launch measured with rocprofv3 (FETCH_SIZE and WRITE_SIZE, each scaled by what
# the same counter reads for a plain 1 GiB device copy), one table per workload and one row per
# kernel, keyed by a digest of the kernel's source so that a reading taken on an older version of
# a kernel is not reported.
TRAFFIC_DIR = os.path.join(ROOT, "profiles")


def traffic_table(workload: str) -> str:
    return os.path.join(TRAFFIC_DIR, f"hbm_traffic_{workload}.md")


KERNEL_SOURCE = {"quantize": "quantize.hip",
                 "chunk_state": "chunk_state.hip", "state_scan": "chunk_state.hip",
                 "state_passing": "state_passing.hip",
                 "chunk_output": "chunk_output.hip", "state_update": "state_update.hip",
                 "state_update_f16": "state_update.hip", "state_update_i8": "state_update.hip",
                 "frontend": "quantize.hip", "frontend (dt softplus)": "quantize.hip",
                 "frontend_step": "quantize.hip"}


def _code_only(text: str) -> str:
    """The source without its comments and blank lines: editing a comment does not change the
    kernel, so it does not void a counter reading."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for f in (KERNEL_SOURCE[kernel], "ssdq_internal.h"):
        with open(os.path.join(ROOT, "quantized_selective_state_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def _sum_or_none(*vals):
    return None if any(v is None for v in vals) else sum(vals)


def measured_traffic(kernel: str, workload: str):
    """Counter-measured HBM bytes per launch of `kernel` on `workload`, or None if the workload's
    table has no row for the kernel's current source."""
    try:
        with open(traffic_table(workload)) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    digest = source_digest(kernel)
    for ln in lines:
        cells = [c.strip() for c in ln.strip().strip("|").split("|")]
        if len(cells) >= 4 and cells[0] == kernel and cells[1] == digest:
            try:
                return int(cells[-1])
            except ValueError:
                return None
    return None


class HipEvent:
    """A HIP timing event created with hipEventDisableSystemFence: recording it does not write back
    and invalidate the caches (a default event's system-scope release does, which costs a few
    microseconds per record and leaves the next kernel with cold caches).  Elapsed times are read
    only after a device synchronisation."""

    _hip = None
    FLAGS = 0x20000000   # hipEventDisableSystemFence

    @classmethod
    def hip(cls):
        if cls._hip is None:
            import ctypes
            lib = ctypes.CDLL("libamdhip64.so.7")   # the runtime torch already loaded (same soname)
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = lib
        return cls._hip

    def __init__(self, stream: int):
        import ctypes
        self.stream = ctypes.c_void_p(stream)
        self.h = ctypes.c_void_p()
        rc = self.hip().hipEventCreateWithFlags(ctypes.byref(self.h), self.FLAGS)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self):
        rc = self.hip().hipEventRecord(self.h, self.stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end: "HipEvent") -> float:
        import ctypes
        ms = ctypes.c_float()
        rc = self.hip().hipEventElapsedTime(ctypes.byref(ms), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.h:
            self._hip.hipEventDestroy(self.h)


PREFILL_WORKLOADS = ["tiny", "mamba2-1.3b-prefill", "mamba2-2.7b-long-prefill", "mamba2-8b-prefill"]
LATENCY_ONLY = {"tiny"}   # a 16 KiB state: bound by launch latency, reported by its latency alone
HEADLINE = "mamba2-8b-prefill"     # the largest prefill configuration that fits one GPU


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--workload", choices=PREFILL_WORKLOADS, action="append",
                    help="prefill workload(s) to run (default: all three, the 8B-shaped one as the headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-frontend", action="store_true")
    ap.add_argument("--no-scale-layouts", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (for scaling HBM counter readings)")
    return ap.parse_args(argv)


def kernel_bytes(b, L, H, P, N, G, Q):
    """Compulsory HBM bytes per launch of each prefill kernel as built: every input read once,
    every output written once (the carried state as two int8 limbs plus a row scale)."""
    nc = -(-L // Q)
    tok = b * L
    x = tok * H * P
    bc = tok * G * N
    dt = tok * H * 4
    acs = b * H * nc * Q * 4
    st32 = b * nc * H * P * N * 4          # chunk states, fp32
    st16 = b * nc * H * P * N * 2 + b * nc * H * P * 4   # carried state: two int8 limbs + row scales
    hfin = b * H * P * N * 4
    # the state stages write Acs and dt in chunk order (each b H nc Q fp32); the output stage reads
    # both from there
    return {
        "quantize": 3 * x + 6 * bc,            # x, B and C in one launch: fp16 in, int8 out
        "chunk_state": x + bc + dt + 2 * acs + st32,
        "state_passing": st32 + acs // Q * 1 + st16 + hfin,
        "chunk_output": x + 2 * bc + 2 * acs + st16 + 2 * tok * H * P,
        # stages 0 + 1 in one kernel: chunk states stay on chip
        "state_scan": x + bc + dt + 2 * acs + st16 + hfin,
    }


def specified_bytes_per_token(H, P, N, G, Q):
    """Per-token compulsory traffic of the four steps of the chunked scan as the scan is specified
    (int8 x, B, C in; fp32 dt, Acs and chunk states; fp16 y out): the unit figures the roofline
    of each step is quoted against.  chunk_scan (the output step) reads x, B, C, dt, Acs and the
    fp32 state entering the chunk (H P N values per chunk of Q tokens) and writes y."""
    return {
        "quantize": 3 * H * P + 6 * G * N,
        "chunk_state": H * P + G * N + 4 * H + 4 * H + 4 * H * P * N / Q,
        "chunk_scan": H * P + 2 * G * N + 4 * H + 4 * H + 4 * H * P * N / Q + 2 * H * P,
    }


def scan_ops(b, L, H, P, N, G, Q):
    """Algorithmic contraction ops (2 per multiply-add) of the chunked scan: chunk
    states, causal C.B^T once per group, causal M.x and C.Hprev per head."""
    nc = -(-L // Q)
    pairs = 0
    for c in range(nc):
        q = min(Q, L - c * Q)
        pairs += q * (q + 1) // 2
    state = 2 * b * L * H * P * N
    cb = 2 * b * G * pairs * N
    mx = 2 * b * H * pairs * P
    ch = 2 * b * L * H * P * N
    return {"chunk_state": state, "chunk_output": cb + mx + ch, "cb_int8": cb}


def bench_prefill(name, steps, warmup, torch, ssdq, workloads, dev, keep_inputs=False):
    """One workload's prefill step (batched quantize of x, B, C + the chunked scan), timed over
    `steps` back-to-back steps after `warmup` untimed ones.  Returns the workload's record (and
    the seeded inputs when keep_inputs)."""
    T = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    print(f"[bench] generating {name}", file=sys.stderr, flush=True)
    inp = workloads.make_prefill(name)
    b, L, H, P, N, G, Q = (inp[k] for k in ("batch", "seqlen", "nheads", "headdim", "dstate", "ngroups", "chunk"))
    x16, B16, C16 = T(inp["x16"]), T(inp["B16"]), T(inp["C16"])
    sx, sB, sC = T(inp["x_scale"]), T(inp["B_scale"]), T(inp["C_scale"])
    dt, A, D, h0 = T(inp["dt"]), T(inp["A"]), T(inp["D"]), T(inp["h0"])
    if not keep_inputs:
        del inp
        inp = None
    qx = torch.empty(x16.shape, dtype=torch.int8, device=dev)
    qB = torch.empty(B16.shape, dtype=torch.int8, device=dev)
    qC = torch.empty(C16.shape, dtype=torch.int8, device=dev)
    buf = ssdq.ScanBuffers(qx, sx, qB, sB, qC, sC, dt, A, D, h0, chunk=Q)

    # With at least one (batch, head) sequence per CU, stage 0 also carries the state across
    # chunks and stage 1 has nothing to launch; the step then runs stages 0 and 2 only.
    fused = ssdq.chunk_scan_state_fused(b, H)
    stages = [0, 2] if fused else [0, 1, 2]
    stage_name = {0: "state_scan" if fused else "chunk_state", 1: "state_passing", 2: "chunk_output"}
    scan_names = [stage_name[st] for st in stages]
    names = ["quantize"] + scan_names

    # x, B and C are quantized by one batched launch
    quant = ssdq.QuantizeBatch([ssdq.QuantizeCall(x16, sx, qx), ssdq.QuantizeCall(B16, sB, qB),
                                ssdq.QuantizeCall(C16, sC, qC)])
    fns = [quant.run] + [(lambda st=st: buf.run_stage(st)) for st in stages]

    def step(marks=None):
        """One pass of the hot path; marks maps a kernel index to (event before, event after)."""
        for i, f in enumerate(fns):
            if marks and i in marks:
                marks[i][0].record()
            f()
            if marks and i in marks:
                marks[i][1].record()

    stream = torch.cuda.current_stream().cuda_stream   # the stream every kernel is launched on
    ev = lambda: HipEvent(stream)
    print(f"[bench] {name}: warmup {warmup}", file=sys.stderr, flush=True)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # per-kernel breakdown: 200 steps with events around every kernel, whatever the timed step
    # count, so that the per-kernel figures average the same number of steps in a short run as
    # in a long one (an event between two kernels can delay the second, so these steps are not
    # the ones whose wall time gives the throughput)
    nprof = 200
    prof = [{i: (ev(), ev()) for i in range(len(fns))} for _ in range(nprof)]
    for k in range(nprof):
        step(prof[k])
    torch.cuda.synchronize()
    per_kernel_ms = {n: sum(prof[k][i][0].elapsed_time(prof[k][i][1]) for k in range(nprof)) / nprof
                     for i, n in enumerate(names)}
    dominant = max(names, key=lambda n: per_kernel_ms[n])
    di = names.index(dominant)

    # timed region: exactly `steps` steps; events only around the dominant kernel (its live
    # launch duration for the roofline) and around the whole region, all on the launch stream
    # (torch's current stream)
    print(f"[bench] {name}: {steps} timed steps", file=sys.stderr, flush=True)
    marks = [{di: (ev(), ev())} for _ in range(steps)]
    e_start, e_end = ev(), ev()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record()
    for k in range(steps):
        step(marks[k])
    e_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_ms = sum(m[di][0].elapsed_time(m[di][1]) for m in marks) / steps
    ms_per_step = wall * 1e3 / steps
    tokens = b * L
    scan_ms = sum(per_kernel_ms[n] for n in scan_names)

    kb = kernel_bytes(b, L, H, P, N, G, Q)
    unit = specified_bytes_per_token(H, P, N, G, Q)
    # the roofline of the dominant kernel, priced by the specified per-token traffic of its step
    # (the output kernel is the chunk_scan step; the others are priced by their own bytes)
    spec_name = {"chunk_output": "chunk_scan", "quantize": "quantize", "chunk_state": "chunk_state"}.get(dominant)
    alg = unit[spec_name] * tokens if spec_name else kb[dominant]
    ach = alg / (dom_ms / 1e3) / 1e9
    own = kb[dominant] / (dom_ms / 1e3) / 1e9
    ops = scan_ops(b, L, H, P, N, G, Q)
    kernels = {n: {"us": round(per_kernel_ms[n] * 1e3, 2),
                   "alg_bytes": kb[n],
                   "alg_GBs": round(kb[n] / (per_kernel_ms[n] / 1e3) / 1e9, 1),
                   "hbm_frac": round(kb[n] / (per_kernel_ms[n] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                   "traffic": measured_traffic(n, name)} for n in names}
    total_ops = ops["chunk_state"] + ops["chunk_output"]   # the state contraction is the same in both plans
    rec = {
        "workload": name, "batch": b, "seqlen": L, "nheads": H, "headdim": P, "dstate": N, "ngroups": G,
        "chunk": Q, "tokens": tokens, "h0": h0 is not None,
        "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "tokens_per_s": round(tokens / (ms_per_step / 1e3), 1),
        "event_ms_per_step": round(e_start.elapsed_time(e_end) / steps, 5),
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(dominant, name), "kernel_us": round(dom_ms * 1e3, 2),
                     "bytes_per_token": unit[spec_name] if spec_name else kb[dominant] / tokens,
                     "units_per_launch": tokens,
                     "kernel_alg_bytes": kb[dominant], "kernel_alg_frac": round(own / HBM_PEAK_GBS, 4)},
        "plan": ("stage 0 carries the state (state passing folded in), blocks of "
                 f"{ssdq.chunk_scan_plan(b, H)} waves") if fused else "three stages",
        "scan_tokens_per_s": round(tokens / (scan_ms / 1e3), 1),
        "mfma_pct_of_int8_peak": round(100 * total_ops / (scan_ms / 1e3) / INT8_PEAK_OPS, 3),
        "chunk_output_mfma_pct_of_int8_peak": round(
            100 * ops["chunk_output"] / (per_kernel_ms["chunk_output"] / 1e3) / INT8_PEAK_OPS, 3),
        "chunk_output_int8_ceiling_pct": round(
            100 * ops["chunk_output"] / (unit["chunk_scan"] * tokens / (HBM_PEAK_GBS * 1e9)) / INT8_PEAK_OPS, 2),
        "kernels": kernels,
    }
    return rec, inp


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        return 2

    import torch
    import quantized_selective_state_amd as ssdq
    import workloads

    dev = torch.device("cuda:0")
    names = args.workload or PREFILL_WORKLOADS
    head = HEADLINE if HEADLINE in names else names[-1]
    records = {}
    head_inp = None
    # the headline workload runs last, so that its timed steps find the GPU at its working clocks
    # (the other workloads' steps run first), whatever the warm-up count asked for
    for name in [n for n in names if n != head] + [head]:
        steps = args.steps if name == head else max(1, min(args.steps, 200))
        warm = args.warmup if name == head else max(1, min(args.warmup, 50))
        rec, inp = bench_prefill(name, steps, warm, torch, ssdq, workloads, dev,
                                 keep_inputs=(name == head and not args.no_cpu_baseline))
        if name in LATENCY_ONLY and name != head:
            rec["roofline"] = None
            rec["latency_us_per_step"] = round(rec["ms_per_step"] * 1e3, 2)
            rec["note"] = "launch-latency bound (a 16 KiB state): latency only, no roofline fraction"
        records[name] = rec
        if inp is not None:
            head_inp = inp
        torch.cuda.empty_cache()
    h = records[head]
    result = {
        "metric": METRIC,
        "value": h["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded; fp16 activations quantized in the timed step)",
        "config": {"workload": head, "batch": h["batch"], "seqlen": h["seqlen"], "nheads": h["nheads"],
                   "headdim": h["headdim"], "dstate": h["dstate"], "ngroups": h["ngroups"], "chunk": h["chunk"]},
        "roofline": h["roofline"],
    }
    for k in ("plan", "scan_tokens_per_s", "event_ms_per_step", "mfma_pct_of_int8_peak",
              "chunk_output_mfma_pct_of_int8_peak", "chunk_output_int8_ceiling_pct", "kernels"):
        result[k] = h[k]
    result["workloads"] = {n: r for n, r in records.items() if n != head}

    if not args.no_frontend:
        result["frontend"] = bench_frontend(args, torch, ssdq, workloads, dev, head)
    if not args.no_scale_layouts:
        result["scale_layouts"] = bench_scale_layouts(args, torch, ssdq, workloads, dev, head)
    if not args.no_decode:
        result["decode"] = bench_decode(args, torch, ssdq, workloads, dev)

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = n

    if not args.no_cpu_baseline and head_inp is not None:
        result["cpu_baseline"] = cpu_baseline(head_inp, workloads)

    print(json.dumps(result), flush=True)
    return 0


def bench_scale_layouts(args, torch, ssdq, workloads, dev, name):
    """The scan (stages only, codes already in HBM) of one workload under each static scale layout
    and with the output correction, against the plain per-head / per-group layout in the same run:
    B, C scales per (group, state), x scales per (head, channel) from 8 channel clusters, both,
    and all of them with the correction.  The scales are calibrated on the draw itself (timing
    only; parity is the tests' business).  Returns microseconds per scan and the ratio to plain."""
    print(f"[bench] generating {name} for the scale layouts", file=sys.stderr, flush=True)
    inp = workloads.make_prefill(name)
    T = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    b, L, H, P, N, G, Q = (inp[k] for k in ("batch", "seqlen", "nheads", "headdim", "dstate", "ngroups", "chunk"))
    x16, B16, C16 = T(inp["x16"]), T(inp["B16"]), T(inp["C16"])
    dt, A, D, h0 = T(inp["dt"]), T(inp["A"]), T(inp["D"]), T(inp["h0"])
    scales = {"head": (T(inp["x_scale"]), T(inp["B_scale"]), T(inp["C_scale"])),
              "fine": (T(workloads.cluster_channel_scales(inp["x16"], 8)),
                       T(workloads.absmax_scale_per_state(inp["B16"])), T(workloads.absmax_scale_per_state(inp["C16"])))}
    y_corr = T(np.random.default_rng(7).normal(0, 0.01, size=(H, P)).astype(np.float32))
    del inp
    y = torch.empty((b, L, H, P), dtype=torch.float16, device=dev)
    hf = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
    ws = torch.empty(ssdq.chunk_scan_workspace_size(b, L, H, P, N, Q), dtype=torch.uint8, device=dev)
    codes = {}
    for key, (sx, sB, sC) in scales.items():
        codes[key] = (ssdq.quantize(x16, sx), ssdq.quantize(B16, sB), ssdq.quantize(C16, sC))
    del x16, B16, C16
    variants = {"plain": ("head", "head", None), "corrected": ("head", "head", y_corr),
                "bc_per_state": ("head", "fine", None), "x_per_channel": ("fine", "head", None),
                "x_per_channel+bc_per_state": ("fine", "fine", None),
                "x_per_channel+bc_per_state+corrected": ("fine", "fine", y_corr)}
    stream = torch.cuda.current_stream().cuda_stream
    bufs = {}
    for vname, (xk, bk, corr) in variants.items():
        qx, sx = codes[xk][0], scales[xk][0]
        qB, qC = codes[bk][1], codes[bk][2]
        sB, sC = scales[bk][1], scales[bk][2]
        bufs[vname] = ssdq.ScanBuffers(qx, sx, qB, sB, qC, sC, dt, A, D, h0, chunk=Q, y=y, h_final=hf,
                                       workspace=ws, y_corr=corr)
    # warm-up of every variant, then rounds that visit the variants in turn (alternating order), so
    # that clock changes over the run fall on all of them alike
    for _ in range(max(2, min(args.warmup, 10))):
        for buf in bufs.values():
            buf.run()
    torch.cuda.synchronize()
    rounds, per = 6, max(1, min(args.steps, 120) // 6)
    total = {v: 0.0 for v in bufs}
    for r in range(rounds):
        order = list(bufs) if r % 2 == 0 else list(reversed(list(bufs)))
        for vname in order:
            e0, e1 = HipEvent(stream), HipEvent(stream)
            e0.record()
            for _ in range(per):
                bufs[vname].run()
            e1.record()
            torch.cuda.synchronize()
            total[vname] += e0.elapsed_time(e1)
    steps = rounds * per
    out = {v: {"scan_us": round(total[v] * 1e3 / steps, 2)} for v in bufs}
    base = out["plain"]["scan_us"]
    for v in out.values():
        v["vs_plain"] = round(v["scan_us"] / base, 4)
    return {"workload": name, "steps": steps, "note": "scan stages only (codes resident); scales calibrated on "
            "the draw itself, x per (head, channel) from 8 channel clusters", "layouts": out}


def bench_frontend(args, torch, ssdq, workloads, dev, name):
    """The same prefill step with the fused front end in place of the quantize launch: the
    depthwise causal conv1d + SiLU + static quantize of the in-projection output (x, B, C
    channels) and dt = softplus(dt_raw + dt_bias), then the scan.  Times the front end alone
    (events around each launch pair) and the whole step."""
    print(f"[bench] generating {name} front end", file=sys.stderr, flush=True)
    fe = workloads.make_frontend(name)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    b, L, H, P, N, G, Q = (fe[k] for k in ("batch", "seqlen", "nheads", "headdim", "dstate", "ngroups", "chunk"))
    xbc, w, cb = T(fe["xbc16"]), T(fe["conv_w"]), T(fe["conv_b"])
    sx, sB, sC = T(fe["x_scale"]), T(fe["B_scale"]), T(fe["C_scale"])
    raw, dtb, A, D = T(fe["dt_raw"]), T(fe["dt_bias"]), T(fe["A"]), T(fe["D"])
    out = (torch.empty((b, L, H, P), dtype=torch.int8, device=dev),
           torch.empty((b, L, G, N), dtype=torch.int8, device=dev),
           torch.empty((b, L, G, N), dtype=torch.int8, device=dev),
           torch.empty((b, L, H), dtype=torch.float32, device=dev))
    qx, qB, qC, dt = out
    buf = ssdq.ScanBuffers(qx, sx, qB, sB, qC, sC, dt, A, D, None, chunk=Q)
    stages = [0, 2] if ssdq.chunk_scan_state_fused(b, H) else [0, 1, 2]
    front = lambda: ssdq.frontend(xbc, w, cb, sx, sB, sC, raw, dtb, H, P, G, N, out=out)

    def step():
        front()
        for st in stages:
            buf.run_stage(st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    steps = min(args.steps, 500)
    pairs = [(HipEvent(stream), HipEvent(stream)) for _ in range(steps)]
    for e0, e1 in pairs:
        e0.record()
        front()
        e1.record()
        for st in stages:
            buf.run_stage(st)
    torch.cuda.synchronize()
    fe_ms = sum(e0.elapsed_time(e1) for e0, e1 in pairs) / steps
    r0, r1 = HipEvent(stream), HipEvent(stream)
    r0.record()
    for _ in range(steps):
        step()
    r1.record()
    torch.cuda.synchronize()
    step_ms = r0.elapsed_time(r1) / steps
    C = H * P + 2 * G * N
    alg = 3 * b * L * C + 8 * b * L * H + 4 * 5 * C   # fp16 in + int8 out; dt in/out; taps + bias
    gbs = alg / (fe_ms / 1e3) / 1e9
    return {"workload": name, "channels": C, "frontend_us": round(fe_ms * 1e3, 2), "alg_bytes": alg,
            "achieved_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": _sum_or_none(measured_traffic("frontend", name),
                                     measured_traffic("frontend (dt softplus)", name)),
            "step_us": round(step_ms * 1e3, 2), "step_tokens_per_s": round(b * L / (step_ms / 1e3), 1)}


def bench_decode(args, torch, ssdq, workloads, dev):
    name = "mamba2-8b-decode"
    print(f"[bench] generating {name}", file=sys.stderr, flush=True)
    dec = workloads.make_decode(name, steps=args.decode_steps)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    sx, sB, sC = T(dec["x_scale"]), T(dec["B_scale"]), T(dec["C_scale"])
    qx, qB, qC = ssdq.quantize(T(dec["x16"]), sx), ssdq.quantize(T(dec["B16"]), sB), ssdq.quantize(T(dec["C16"]), sC)
    dt, A, D = T(dec["dt"]), T(dec["A"]), T(dec["D"])
    state = T(dec["state"])
    steps = qx.shape[0]
    b, H, P, N = state.shape
    G = qB.shape[2]
    ys = torch.empty((steps, b, H, P), dtype=torch.float16, device=dev)
    for t in range(min(8, steps)):     # warmup (the state keeps evolving; values stay bounded)
        ssdq.state_update(state, qx[t], sx, qB[t], sB, qC[t], sC, dt[t], A, D, y=ys[t])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(steps):
        ssdq.state_update(state, qx[t], sx, qB[t], sB, qC[t], sC, dt[t], A, D, y=ys[t])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    io_bytes = b * H * P + 2 * b * G * N + b * H * 4 + b * H * P * 2   # x codes, B/C codes, dt, y
    per_step = 2 * b * H * P * N * 4 + io_bytes
    gbs = per_step / (ms / 1e3) / 1e9
    out = {"workload": name, "batch": b, "nheads": H, "headdim": P, "dstate": N, "ngroups": G, "steps": steps,
           "us_per_step": round(ms * 1e3, 2), "tokens_per_s": round(b / (ms / 1e3), 1),
           "alg_bytes_per_step": per_step, "achieved_GBs": round(gbs, 1),
           "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic("state_update", name)}

    # the decode front end for the same sequences: conv state (b, 3, channels) fp16, one token
    ch = H * P + 2 * G * N
    gen = torch.Generator(device=dev).manual_seed(7)
    xbc_t = torch.randn((b, ch), generator=gen, device=dev).half()
    conv_state = torch.randn((b, 3, ch), generator=gen, device=dev).half()
    taps = torch.randn((ch, 4), generator=gen, device=dev) * 0.3
    raw_t = torch.randn((b, H), generator=gen, device=dev) - 4.0
    fe_out = (torch.empty((b, H, P), dtype=torch.int8, device=dev), torch.empty((b, G, N), dtype=torch.int8, device=dev),
              torch.empty((b, G, N), dtype=torch.int8, device=dev), torch.empty((b, H), dtype=torch.float32, device=dev))
    fe_step = lambda: ssdq.frontend_step(conv_state, xbc_t, taps, None, sx, sB, sC, raw_t, None, H, P, G, N, out=fe_out)
    for _ in range(8):
        fe_step()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        fe_step()
    e1.record()
    torch.cuda.synchronize()
    ms_fe = e0.elapsed_time(e1) / steps
    fe_bytes = b * ch * (2 + 2 * 3 * 2 + 1) + b * H * 8 + ch * 16   # token in, state in/out, codes; dt; taps
    out["frontend_step"] = {"us_per_step": round(ms_fe * 1e3, 2), "alg_bytes_per_step": fe_bytes,
                            "achieved_GBs": round(fe_bytes / (ms_fe / 1e3) / 1e9, 1),
                            "hbm_frac": round(fe_bytes / (ms_fe / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                            "traffic": measured_traffic("frontend_step", name)}
    del xbc_t, conv_state

    # the same steps on the state cached in binary16 (half the state bytes per step)
    del state
    state16 = T(dec["state"]).half()
    for t in range(min(8, steps)):
        ssdq.state_update(state16, qx[t], sx, qB[t], sB, qC[t], sC, dt[t], A, D, y=ys[t])
    torch.cuda.synchronize()
    e0.record()
    for t in range(steps):
        ssdq.state_update(state16, qx[t], sx, qB[t], sB, qC[t], sC, dt[t], A, D, y=ys[t])
    e1.record()
    torch.cuda.synchronize()
    ms16 = e0.elapsed_time(e1) / steps
    per_step16 = 2 * b * H * P * N * 2 + io_bytes
    gbs16 = per_step16 / (ms16 / 1e3) / 1e9
    out["f16_state"] = {"us_per_step": round(ms16 * 1e3, 2), "tokens_per_s": round(b / (ms16 / 1e3), 1),
                        "alg_bytes_per_step": per_step16, "achieved_GBs": round(gbs16, 1),
                        "hbm_frac": round(gbs16 / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic("state_update_f16", name)}

    # and on the state cached as 8-bit codes with one fp32 scale per state row (a quarter of the bytes)
    del state16
    st32 = T(dec["state"])
    scale8 = (st32.abs().amax(dim=-1) / 127.0).contiguous()
    state8 = torch.round(st32 / scale8[..., None]).clamp_(-127, 127).to(torch.int8).contiguous()
    del st32
    for t in range(min(8, steps)):
        ssdq.state_update(state8, qx[t], sx, qB[t], sB, qC[t], sC, dt[t], A, D, y=ys[t], state_scale=scale8)
    torch.cuda.synchronize()
    e0.record()
    for t in range(steps):
        ssdq.state_update(state8, qx[t], sx, qB[t], sB, qC[t], sC, dt[t], A, D, y=ys[t], state_scale=scale8)
    e1.record()
    torch.cuda.synchronize()
    ms8 = e0.elapsed_time(e1) / steps
    per_step8 = 2 * (b * H * P * N + b * H * P * 4) + io_bytes
    gbs8 = per_step8 / (ms8 / 1e3) / 1e9
    out["i8_state"] = {"us_per_step": round(ms8 * 1e3, 2), "tokens_per_s": round(b / (ms8 / 1e3), 1),
                       "alg_bytes_per_step": per_step8, "achieved_GBs": round(gbs8, 1),
                       "hbm_frac": round(gbs8 / HBM_PEAK_GBS, 4),
                       "traffic": measured_traffic("state_update_i8", name)}
    return out


def _cpu_model() -> str:
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return cpu


def cpu_baseline(inp, workloads):
    """The oracle as it stands (quantizer + fp64 sequential recurrence) on the host cores: the
    whole headline workload (every (batch, head) sequence) once on all available threads, and a
    sample of the 1.3B-shaped workload on one thread."""
    import oracle
    threads = oracle.default_threads()
    print(f"[bench] cpu oracle on {threads} threads", file=sys.stderr, flush=True)
    # whole-workload runs repeated until about 10 s of host time have passed (at most 3)
    runs, t0 = 0, time.perf_counter()
    while runs < 3 and (runs == 0 or time.perf_counter() - t0 < 10.0):
        codes = oracle.codes_from_inputs(inp)
        oracle.ssd(codes, threads=threads)
        del codes
        runs += 1
    sec = (time.perf_counter() - t0) / runs
    tokens = inp["batch"] * inp["seqlen"]
    seqs = inp["batch"] * inp["nheads"]
    # one thread: the first 64 heads of batch 0 of the 1.3B-shaped workload, scaled to the whole
    # workload's tokens
    name1 = "mamba2-1.3b-prefill"
    print(f"[bench] cpu oracle on 1 thread, {name1} sample", file=sys.stderr, flush=True)
    small = workloads.make_prefill(name1)
    c1 = oracle.codes_from_inputs(small)
    k = 64
    t1 = time.perf_counter()
    oracle.ssd(c1, pairs=[(0, h) for h in range(k)], threads=1)
    sec1 = time.perf_counter() - t1
    seqs1 = small["batch"] * small["nheads"]
    tok1 = small["batch"] * small["seqlen"]
    return {"value": round(tokens / sec, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"whole workload: quantize x,B,C + all {seqs} (batch, head) sequences of {inp['seqlen']} "
                      f"tokens, fp64; {runs} runs, {sec:.2f} s each",
            "cpu": _cpu_model(), "nproc": os.cpu_count(), "threads_available": threads,
            "one_thread": {"workload": name1, "value": round(tok1 / (sec1 * seqs1 / k), 1), "unit": "tokens/s",
                           "sample": f"{k} of {seqs1} (batch, head) sequences of {small['seqlen']} tokens, "
                                     f"{sec1:.2f} s, scaled to the whole workload"}}


if __name__ == "__main__":
    sys.exit(main())
