"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
HIP path through the C ABI binding, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

Y_TOL = 2e-3      # max|y - y_ref| <= Y_TOL * max|y_ref|
H_TOL = 1e-4      # max|h - h_ref| <= H_TOL * max|h_ref|


def dev() -> torch.device:
    return torch.device("cuda:0")


def to_dev(a):
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    mask = np.isfinite(ref)
    if not np.all(np.isfinite(got[mask])):
        return float("inf")
    scale = np.max(np.abs(ref[mask])) if mask.any() else 0.0
    return float(np.max(np.abs(got[mask] - ref[mask])) / max(scale, 1e-300))


def gpu_quantize_inputs(inp: dict):
    """Quantize x, B, C on the GPU; returns device codes and scales."""
    import quantized_selective_state_amd as ssdq
    sx, sB, sC = to_dev(inp["x_scale"]), to_dev(inp["B_scale"]), to_dev(inp["C_scale"])
    qx = ssdq.quantize(to_dev(inp["x16"]), sx)
    qB = ssdq.quantize(to_dev(inp["B16"]), sB)
    qC = ssdq.quantize(to_dev(inp["C16"]), sC)
    return qx, sx, qB, sB, qC, sC


def gpu_prefill(inp: dict, chunk: int | None = None, with_D=True, with_h0=True):
    """GPU quantize + chunk scan.  Returns (codes dict (numpy), y (numpy f32), h_final (numpy))."""
    import quantized_selective_state_amd as ssdq
    qx, sx, qB, sB, qC, sC = gpu_quantize_inputs(inp)
    h0 = to_dev(inp["h0"]) if with_h0 else None
    D = to_dev(inp["D"]) if with_D else None
    y, hf = ssdq.chunk_scan(qx, sx, qB, sB, qC, sC, to_dev(inp["dt"]), to_dev(inp["A"]), D, h0,
                            chunk=chunk or inp["chunk"])
    torch.cuda.synchronize()
    codes = dict(qx=qx.cpu().numpy(), qB=qB.cpu().numpy(), qC=qC.cpu().numpy())
    return codes, y.float().cpu().numpy(), hf.cpu().numpy()


def oracle_codes(inp: dict, with_D=True, with_h0=True) -> oracle.Codes:
    c = oracle.codes_from_inputs(inp)
    if not with_D:
        c.D = None
    if not with_h0:
        c.h0 = None
    return c


def threaded(fn, items, threads: int | None = None) -> list:
    """fn over items on host threads (the oracle's C calls release the interpreter lock)."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(threads or oracle.default_threads()) as ex:
        return list(ex.map(fn, items))


def compare_full(c: "oracle.Codes", y_of, h_of, tag: str, state_f16: bool = False, y_tol: float = Y_TOL,
                 h_tol: float = H_TOL) -> dict:
    """Every (batch, head) sequence of a workload against the oracle, one batch index at a time
    (so that only one batch index of the fp64 reference is held in memory).  y_of(b) gives the
    GPU's y of batch index b as a host array (L, H, P) and h_of(b) its final state (H, P, N).
    Asserts the whole-tensor bars max|y - y_ref| <= y_tol max|y_ref| and max|h - h_ref| <=
    h_tol max|h_ref|, and reports the worst single-sequence ratios as a diagnostic (a global
    maximum can hide a small head next to an outlier head)."""
    ey = ymax = eh = hmax = 0.0
    worst_y = worst_h = (0.0, None)
    for b in range(c.batch):
        y_ref, h_ref = oracle.ssd_batch(c, b, state_f16=state_f16)
        yg = np.asarray(y_of(b), dtype=np.float64)
        hg = np.asarray(h_of(b), dtype=np.float64)
        assert yg.shape == y_ref.shape and hg.shape == h_ref.shape
        assert np.all(np.isfinite(yg)) and np.all(np.isfinite(hg)), f"{tag}: non-finite output at batch {b}"
        dy = np.abs(yg - y_ref).max(axis=(0, 2))            # per head
        ry = np.abs(y_ref).max(axis=(0, 2))
        dh = np.abs(hg - h_ref).max(axis=(1, 2))
        rh = np.abs(h_ref).max(axis=(1, 2))
        ey, ymax = max(ey, float(dy.max())), max(ymax, float(ry.max()))
        eh, hmax = max(eh, float(dh.max())), max(hmax, float(rh.max()))
        with np.errstate(divide="ignore", invalid="ignore"):
            sy = np.where(ry > 0, dy / ry, np.where(dy > 0, np.inf, 0.0))
            sh = np.where(rh > 0, dh / rh, np.where(dh > 0, np.inf, 0.0))
        h = int(np.argmax(sy))
        if sy[h] >= worst_y[0]:
            worst_y = (float(sy[h]), (b, h))
        h = int(np.argmax(sh))
        if sh[h] >= worst_h[0]:
            worst_h = (float(sh[h]), (b, h))
    out = dict(y_err=ey / max(ymax, 1e-300), h_err=eh / max(hmax, 1e-300), worst_seq_y=worst_y,
               worst_seq_h=worst_h, sequences=c.batch * c.H)
    note(f"{tag}: all {out['sequences']} sequences: y_err={out['y_err']:.3e} h_err={out['h_err']:.3e}; "
         f"worst single-sequence ratio y {worst_y[0]:.3e} at (b, h) = {worst_y[1]}, "
         f"h {worst_h[0]:.3e} at {worst_h[1]}")
    assert out["y_err"] <= y_tol, out
    assert out["h_err"] <= h_tol, out
    return out


def carried_state(hprev: np.ndarray, hscale: np.ndarray) -> np.ndarray:
    """The state entering each chunk from the workspace's two INT8 limbs and row scales,
    (..., 2, P, N) int8 + (..., P) fp32 -> (..., P, N) fp64.  Full 64-state blocks of a row are
    stored with their 4-byte groups transposed (state 64 blk + 16 t + 4 k + i at
    64 blk + 16 k + 4 t + i); a partial last block is in natural order."""
    N = hprev.shape[-1]
    nat = hprev.astype(np.float64).copy()
    for blk in range(N // 64):
        sl = hprev[..., 64 * blk:64 * blk + 64].astype(np.float64)
        g = sl.reshape(sl.shape[:-1] + (4, 4, 4))          # stored (k, t, i)
        nat[..., 64 * blk:64 * blk + 64] = np.swapaxes(g, -3, -2).reshape(sl.shape)   # natural (t, k, i)
    return (nat[..., 0, :, :] + nat[..., 1, :, :] / 256.0) * hscale[..., None].astype(np.float64)
