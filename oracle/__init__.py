"""CPU oracle for the INT8-input Mamba-2 SSD scan -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may use
this package.  It wraps liboracle.so (built from ssd_oracle.c with gcc) and
shares nothing with the HIP library.  See ssd_oracle.c for what each function
computes and which passage of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A different build of the same source (the planted-mistake test points the pins at mutated
# copies of the oracle through this variable); unset, the library next to the source is used.
_LIB_OVERRIDE = os.environ.get("SSD_ORACLE_LIB")
_lib = None


def compile_library(src: str, out: str, verbose: bool = False) -> str:
    """Compile an oracle source file to a shared library with gcc (strict IEEE: no fast-math,
    no contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
           "-Wall", "-Wextra", src, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False) -> str:
    """Compile liboracle.so from ssd_oracle.c."""
    return compile_library(_SRC, _LIB, verbose)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.oracle_quantize_f16.argtypes = [P, P, P, i64, i32, i32]
    lib.oracle_quantize_f16.restype = None
    lib.oracle_ssd_sequential.argtypes = [P] * 10 + [i32, i64, i32, i32, i32, i32, i32, i32, P, P, i32, P, P, i32]
    lib.oracle_ssd_sequential.restype = None
    lib.oracle_ssd_sequential_state_f16.argtypes = [P] * 10 + [i32, i64, i32, i32, i32, i32, i32, i32, P, P, P, i32]
    lib.oracle_ssd_sequential_state_f16.restype = None
    lib.oracle_round_binary16.argtypes = [P, P, i64]
    lib.oracle_frontend.argtypes = [P, P, P, i32, i32, i64, i32, P, P, P]
    lib.oracle_frontend.restype = None
    lib.oracle_softplus_dt.argtypes = [P, P, i64, i32, P]
    lib.oracle_softplus_dt.restype = None
    lib.oracle_requantize_rows_i8.argtypes = [P, i64, i32, P, P, P]
    lib.oracle_requantize_rows_i8.restype = None
    lib.oracle_ssd_sequential_state_i8.argtypes = [P] * 11 + [i32, i64, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, i32]
    lib.oracle_ssd_sequential_values.argtypes = [P] * 7 + [i32, i64, i32, i32, i32, i32, i32, i32, P, P]
    lib.oracle_ssd_sequential_values.restype = None
    lib.oracle_ssd_sequential_state_i8.restype = None
    lib.oracle_round_binary16.restype = None
    lib.oracle_chunk_cumsum.argtypes = [P, P, i64, i32, i32, i32, i32, P]
    lib.oracle_chunk_cumsum.restype = None
    lib.oracle_chunk_state.argtypes = [P] * 6 + [i64, i32, i32, i32, i32, i32, i32, i32, P, i32]
    lib.oracle_quantize_f16_per_channel.argtypes = [P, P, P, i64, i32, i32]
    lib.oracle_quantize_f16_per_channel.restype = None
    lib.oracle_chunk_state.restype = None
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# ----------------------------------------------------------------------------------------------
# quantizer


def quantize(x16: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Codes of an fp16 tensor whose second-to-last axis indexes `scale`
    (heads for x (..., H, P); groups for B/C (..., G, N))."""
    lib = _load()
    x16 = np.ascontiguousarray(x16, dtype=np.float16)
    scale = _c(scale, np.float32)
    nscale, inner = x16.shape[-2], x16.shape[-1]
    assert scale.shape == (nscale,)
    rows = x16.size // (nscale * inner) if x16.size else 0
    q = np.empty(x16.shape, dtype=np.int8)
    if x16.size:
        lib.oracle_quantize_f16(_ptr(x16.view(np.uint16)), _ptr(q), _ptr(scale), rows, nscale, inner)
    return q


def quantize_per_channel(x16: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Codes of an fp16 tensor (..., K, I) with one scale per (k, i): scale (K, I) (B or C with a
    scale per (group, state))."""
    lib = _load()
    x16 = np.ascontiguousarray(x16, dtype=np.float16)
    scale = _c(scale, np.float32)
    nscale, inner = x16.shape[-2], x16.shape[-1]
    assert scale.shape == (nscale, inner)
    rows = x16.size // (nscale * inner) if x16.size else 0
    q = np.empty(x16.shape, dtype=np.int8)
    if x16.size:
        lib.oracle_quantize_f16_per_channel(_ptr(x16.view(np.uint16)), _ptr(q), _ptr(scale), rows, nscale, inner)
    return q


def quantize_values(v16: np.ndarray, scale: float) -> np.ndarray:
    """Codes of a flat fp16 array under one scale."""
    v16 = np.ascontiguousarray(v16, dtype=np.float16).reshape(-1, 1, 1)
    return quantize(v16, np.array([scale], dtype=np.float32)).reshape(-1)


# ----------------------------------------------------------------------------------------------
# recurrence


class Codes:
    """Quantized prefill inputs in the scan's layout; y_corr (H, P) float32 is the optional output
    correction added to every y.  sx is one scale per head (H,) or one per (head, channel)
    (H, P); sB and sC are one scale per group (G,) or one per (group, state) (G, N)."""

    def __init__(self, qx, sx, qB, sB, qC, sC, dt, A, D=None, h0=None, y_corr=None):
        self.qx = _c(qx, np.int8)
        self.qB = _c(qB, np.int8)
        self.qC = _c(qC, np.int8)
        self.sx, self.sB, self.sC = _c(sx, np.float32), _c(sB, np.float32), _c(sC, np.float32)
        self.dt, self.A = _c(dt, np.float32), _c(A, np.float32)
        self.D, self.h0 = _c(D, np.float32), _c(h0, np.float32)
        self.y_corr = _c(y_corr, np.float32)
        self.batch, self.L, self.H, self.P = self.qx.shape
        assert self.y_corr is None or self.y_corr.shape == (self.H, self.P)
        self.G, self.N = self.qB.shape[2], self.qB.shape[3]
        assert self.qB.shape == (self.batch, self.L, self.G, self.N) == self.qC.shape
        assert self.dt.shape == (self.batch, self.L, self.H)
        assert self.H % self.G == 0
        assert self.sB.shape == self.sC.shape and self.sB.shape in ((self.G,), (self.G, self.N))
        assert self.sx.shape in ((self.H,), (self.H, self.P))
        self.per_state = int(self.sB.shape == (self.G, self.N))
        self.x_per_channel = int(self.sx.shape == (self.H, self.P))

    @property
    def scale_flags(self) -> int:
        """The oracle's scale-layout word: bit 0 B, C per (group, state); bit 1 x per (head, channel)."""
        return int(self.per_state) | (int(self.x_per_channel) << 1)


def _quantize_bc(t16: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Codes under one scale per row group (1-D scale) or one per (group, element) (2-D)."""
    return quantize_per_channel(t16, scale) if np.ndim(scale) == 2 else quantize(t16, scale)


def codes_from_inputs(inp: dict) -> Codes:
    """Quantize a workload draw with the oracle's quantizer (with its output correction y_corr,
    if the draw carries one; x scales per head (H,) or per (head, channel) (H, P); B and C scales
    per group (G,) or per (group, state) (G, N))."""
    return Codes(_quantize_bc(inp["x16"], inp["x_scale"]), inp["x_scale"],
                 _quantize_bc(inp["B16"], inp["B_scale"]), inp["B_scale"],
                 _quantize_bc(inp["C16"], inp["C_scale"]), inp["C_scale"],
                 inp["dt"], inp["A"], inp.get("D"), inp.get("h0"), inp.get("y_corr"))


def ssd_one(c: Codes, b: int, h: int, chunk: int = 0, state_f16: bool = False):
    """(y (L,P), h_final (P,N), bounds (nc,P,N) or None) for one (b, h) in float64.  With
    state_f16 the state is cached in binary16 between tokens (no chunk bounds then)."""
    lib = _load()
    y = np.empty((c.L, c.P), np.float64)
    hf = np.empty((c.P, c.N), np.float64)
    if state_f16:
        lib.oracle_ssd_sequential_state_f16(_ptr(c.qx), _ptr(c.sx), _ptr(c.qB), _ptr(c.sB), _ptr(c.qC), _ptr(c.sC),
                                            _ptr(c.dt), _ptr(c.A), _ptr(c.D), _ptr(c.h0),
                                            c.batch, c.L, c.H, c.P, c.N, c.G, b, h, _ptr(y), _ptr(hf),
                                            _ptr(c.y_corr), c.scale_flags)
        return y, hf, None
    bounds = None
    if chunk > 0:
        bounds = np.empty(((c.L + chunk - 1) // chunk, c.P, c.N), np.float64)
    lib.oracle_ssd_sequential(_ptr(c.qx), _ptr(c.sx), _ptr(c.qB), _ptr(c.sB), _ptr(c.qC), _ptr(c.sC),
                              _ptr(c.dt), _ptr(c.A), _ptr(c.D), _ptr(c.h0),
                              c.batch, c.L, c.H, c.P, c.N, c.G, b, h, _ptr(y), _ptr(hf),
                              chunk, _ptr(bounds), _ptr(c.y_corr), c.scale_flags)
    return y, hf, bounds


def ssd(c: Codes, pairs=None, chunk: int = 0, threads: int | None = None, state_f16: bool = False):
    """Run the recurrence for the given (b, h) pairs (default: all) on `threads` host threads.
    Returns (y, h_final, bounds) as full-size float64 arrays (NaN where not computed),
    bounds only when chunk > 0.  state_f16: the state cached in binary16 between tokens."""
    if pairs is None:
        pairs = [(b, h) for b in range(c.batch) for h in range(c.H)]
    y = np.full((c.batch, c.L, c.H, c.P), np.nan)
    hf = np.full((c.batch, c.H, c.P, c.N), np.nan)
    bounds = None
    if chunk > 0:
        bounds = np.full((c.batch, (c.L + chunk - 1) // chunk, c.H, c.P, c.N), np.nan)
    threads = threads or default_threads()

    def one(bh):
        b, h = bh
        yy, hh, bb = ssd_one(c, b, h, chunk, state_f16)
        y[b, :, h, :] = yy
        hf[b, h] = hh
        if bb is not None:
            bounds[b, :, h] = bb

    if threads <= 1:
        for bh in pairs:
            one(bh)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, pairs))
    return y, hf, bounds


def ssd_batch(c: Codes, b: int, threads: int | None = None, state_f16: bool = False):
    """Every head of batch index b: (y (L, H, P), h_final (H, P, N)) in float64, the heads run
    on `threads` host threads.  Lets a caller compare a whole workload one batch index at a
    time, holding only that much of the reference in memory."""
    y = np.empty((c.L, c.H, c.P), np.float64)
    hf = np.empty((c.H, c.P, c.N), np.float64)
    threads = threads or default_threads()

    def one(h):
        yy, hh, _ = ssd_one(c, b, h, 0, state_f16)
        y[:, h, :] = yy
        hf[h] = hh

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(one, range(c.H)))
    return y, hf


def ssd_one_state_i8(c: Codes, b: int, h: int, q0=None, s0=None, scales_per_step: bool = False):
    """The recurrence for one (b, h) with the state cached as 8-bit codes and one binary32
    scale per state row between tokens, starting from codes q0 (batch,H,P,N) int8 with row
    scales s0 (batch,H,P) float32 (None: a zero state).  Returns (y (L,P), decoded final state
    (P,N), final codes (P,N) int8, final scales (P,) float32, last token's update before
    re-quantization (P,N)), all from the oracle; with scales_per_step also the row scales after
    every token (L,P) float32 as a sixth item."""
    lib = _load()
    y = np.empty((c.L, c.P), np.float64)
    hf = np.empty((c.P, c.N), np.float64)
    q = np.empty((c.P, c.N), np.int8)
    s = np.empty(c.P, np.float32)
    u = np.empty((c.P, c.N), np.float64)
    q0 = None if q0 is None else _c(q0, np.int8)
    s0 = None if s0 is None else _c(s0, np.float32)
    if (q0 is None) != (s0 is None):
        raise ValueError("q0 and s0 go together")
    if q0 is not None and (q0.shape != (c.batch, c.H, c.P, c.N) or s0.shape != (c.batch, c.H, c.P)):
        raise ValueError("q0 must be (batch,H,P,N) and s0 (batch,H,P)")
    steps = np.empty((c.L, c.P), np.float32) if scales_per_step else None
    lib.oracle_ssd_sequential_state_i8(_ptr(c.qx), _ptr(c.sx), _ptr(c.qB), _ptr(c.sB), _ptr(c.qC), _ptr(c.sC),
                                       _ptr(c.dt), _ptr(c.A), _ptr(c.D), _ptr(q0), _ptr(s0),
                                       c.batch, c.L, c.H, c.P, c.N, c.G, b, h, _ptr(y), _ptr(hf), _ptr(q),
                                       _ptr(s), _ptr(u), _ptr(steps), _ptr(c.y_corr), c.scale_flags)
    if scales_per_step:
        return y, hf, q, s, u, steps
    return y, hf, q, s, u


def ssd_values_one(v: dict, b: int, h: int):
    """The recurrence for one (b, h) over real-valued inputs: v holds x (batch, L, H, P), B and C
    (batch, L, G, N) as float64 (for instance the binary16 activations before quantization), dt,
    A, and optionally D and h0.  Returns (y (L, P), h_final (P, N)) in float64."""
    lib = _load()
    x, B, C = _c(v["x"], np.float64), _c(v["B"], np.float64), _c(v["C"], np.float64)
    dt, A = _c(v["dt"], np.float32), _c(v["A"], np.float32)
    D, h0 = _c(v.get("D"), np.float32), _c(v.get("h0"), np.float32)
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.empty((L, P), np.float64)
    hf = np.empty((P, N), np.float64)
    lib.oracle_ssd_sequential_values(_ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(A), _ptr(D), _ptr(h0), batch, L, H,
                                     P, N, G, b, h, _ptr(y), _ptr(hf))
    return y, hf


def mean_correction(inp: dict, threads: int | None = None) -> np.ndarray:
    """SSDi8's per-channel mean correction (its abstract describes a correction derived from error
    statistics gathered per channel; Figure 1b labels it a mean correction), calibrated on a draw `inp` (binary16
    x, B, C with their static scales, dt, A, D, h0) the plainest way the pages support: the error
    of the quantized scan's output channel (h, p) is y_ref - y_q, with y_ref the recurrence over the
    unquantized binary16 inputs and y_q the recurrence over their INT8 codes; the correction is
    its mean over every (batch, token) position of the draw.  Returns y_corr (H, P) float32, the
    term added to every y of the corrected scan."""
    c = codes_from_inputs(inp)
    vals = dict(x=inp["x16"].astype(np.float64), B=inp["B16"].astype(np.float64), C=inp["C16"].astype(np.float64),
                dt=inp["dt"], A=inp["A"], D=inp.get("D"), h0=inp.get("h0"))
    sums = np.zeros((c.batch, c.H, c.P))

    def one(bh):
        b, h = bh
        y_q, _, _ = ssd_one(c, b, h)
        y_ref, _ = ssd_values_one(vals, b, h)
        sums[b, h] = (y_ref - y_q).sum(axis=0)

    with ThreadPoolExecutor(threads or default_threads()) as ex:
        list(ex.map(one, [(b, h) for b in range(c.batch) for h in range(c.H)]))
    return (sums.sum(axis=0) / (c.batch * c.L)).astype(np.float32)


def requantize_rows_i8(rows: np.ndarray):
    """Each row of a (rows, N) array as 8-bit codes with one binary32 scale: (codes, scales,
    decoded rows)."""
    r = _c(np.atleast_2d(rows), np.float64)
    q = np.empty(r.shape, np.int8)
    s = np.empty(r.shape[0], np.float32)
    out = np.empty(r.shape, np.float64)
    _load().oracle_requantize_rows_i8(_ptr(r), r.shape[0], r.shape[1], _ptr(q), _ptr(s), _ptr(out))
    return q, s, out


def frontend(xbc16: np.ndarray, w: np.ndarray, bias, x_scale, B_scale, C_scale, H: int, P: int,
             G: int, N: int) -> dict:
    """The block's front end on (batch, L, H*P + 2*G*N) binary16 activations: the convolution +
    bias (`pre`), SiLU of it (`act`, unrounded), the binary16 module output (`act16`), and the
    static INT8 codes of its x, B and C slices (`qx` (b,L,H,P), `qB`, `qC` (b,L,G,N))."""
    x = _c(xbc16, np.float16)
    b, L, C = x.shape
    if C != H * P + 2 * G * N:
        raise ValueError("channels must be H*P + 2*G*N")
    w = _c(w, np.float32)
    dconv = w.shape[1]
    bias = _c(bias, np.float32)
    pre = np.empty((b, L, C), np.float64)
    act = np.empty((b, L, C), np.float64)
    a16 = np.empty((b, L, C), np.float64)
    _load().oracle_frontend(_ptr(x.view(np.uint16)), _ptr(w), _ptr(bias), dconv, b, L, C, _ptr(pre), _ptr(act),
                            _ptr(a16))
    act16 = a16.astype(np.float16)          # exact: every value is a binary16 value
    hp, gn = H * P, G * N
    return dict(pre=pre, act=act, act16=act16,
                qx=quantize(act16[..., :hp].reshape(b, L, H, P), x_scale),
                qB=quantize(act16[..., hp:hp + gn].reshape(b, L, G, N), B_scale),
                qC=quantize(act16[..., hp + gn:].reshape(b, L, G, N), C_scale))


def softplus_dt(dt_raw: np.ndarray, dt_bias) -> np.ndarray:
    """softplus(dt_raw + dt_bias[h]) in float64; dt_raw (..., H)."""
    d = _c(dt_raw, np.float32)
    H = d.shape[-1]
    out = np.empty(d.shape, np.float64)
    _load().oracle_softplus_dt(_ptr(d), _ptr(_c(dt_bias, np.float32)), d.size // H, H, _ptr(out))
    return out


def round_binary16(v: np.ndarray) -> np.ndarray:
    """The binary16 value nearest to each element (ties to even), as float64."""
    lib = _load()
    src = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty_like(src)
    lib.oracle_round_binary16(_ptr(src), _ptr(out), src.size)
    return out


def chunk_cumsum(c: Codes, b: int, h: int, chunk: int) -> np.ndarray:
    lib = _load()
    nc = (c.L + chunk - 1) // chunk
    out = np.full(nc * chunk, np.nan)
    lib.oracle_chunk_cumsum(_ptr(c.dt), _ptr(c.A), c.L, c.H, b, h, chunk, _ptr(out))
    return out.reshape(nc, chunk)


def chunk_state(c: Codes, b: int, h: int, chunk: int) -> np.ndarray:
    lib = _load()
    nc = (c.L + chunk - 1) // chunk
    out = np.empty((nc, c.P, c.N))
    lib.oracle_chunk_state(_ptr(c.qx), _ptr(c.sx), _ptr(c.qB), _ptr(c.sB), _ptr(c.dt), _ptr(c.A),
                           c.L, c.H, c.P, c.N, c.G, b, h, chunk, _ptr(out), c.scale_flags)
    return out


def decode_as_prefill(dec: dict) -> Codes:
    """The decode workload as one prefill over its steps: the recurrence is the
    same, with the decode state as h0.  Codes come from the oracle quantizer."""
    qx = _quantize_bc(dec["x16"], dec["x_scale"])      # (T, b, H, P)
    qB = _quantize_bc(dec["B16"], dec["B_scale"])      # (T, b, G, N)
    qC = _quantize_bc(dec["C16"], dec["C_scale"])
    tr = lambda a: np.ascontiguousarray(np.swapaxes(a, 0, 1))
    return Codes(tr(qx), dec["x_scale"], tr(qB), dec["B_scale"], tr(qC), dec["C_scale"],
                 tr(dec["dt"]), dec["A"], dec["D"], dec["state"])
