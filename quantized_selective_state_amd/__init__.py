"""Python binding of libssdq, the INT8-input Mamba-2 SSD scan for MI355X (gfx950).

The functions below only marshal arguments: they check device, dtype, shape and
contiguity of torch tensors, pass their device pointers and the current HIP
stream to the C ABI declared in include/ssdq.h, and raise on a non-success
status.  Every step of the computation runs in the library's HIP kernels;
torch only provides device memory and the stream.  There is no fallback: if
libssdq.so is missing, importing this package fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssdq.so")

SSDQ_SUCCESS = 0
SSDQ_ERROR_INVALID_VALUE = 1
SSDQ_ERROR_UNSUPPORTED = 2
SSDQ_ERROR_WORKSPACE_TOO_SMALL = 3
SSDQ_ERROR_LAUNCH = 4
SSDQ_ERROR_SCRATCH_LIMIT = 5
NOALLOC_SCRATCH_BYTES = 64 << 20
CHUNK_SCAN_STAGES = 3
STAGE_NAMES = ("chunk_state", "state_passing", "chunk_output")   # stage 0 also runs the chunk cumsum

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python quantized_selective_state_amd/build.py` "
                      "(or __graft_entry__.build())")

lib = ctypes.CDLL(LIB_PATH)
_P, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t

lib.ssdq_status_string.argtypes = [ctypes.c_int]
lib.ssdq_status_string.restype = ctypes.c_char_p
lib.ssdq_quantize.argtypes = [_P, _P, _P, _i64, _i32, _i32, _P]
lib.ssdq_quantize.restype = ctypes.c_int


class QuantizeJob(ctypes.Structure):
    """ssdq_quantize_job: the arguments of one ssdq_quantize call."""
    _fields_ = [("x_f16", _P), ("q", _P), ("scale", _P), ("rows", _i64), ("nscale", _i32), ("inner", _i32)]


QUANTIZE_MAX_JOBS = 8
lib.ssdq_quantize_batch.argtypes = [ctypes.POINTER(QuantizeJob), _i32, _P]
lib.ssdq_quantize_batch.restype = ctypes.c_int
lib.ssdq_chunk_scan_workspace_size.argtypes = [_i32, _i64, _i32, _i32, _i32, _i32]
lib.ssdq_chunk_scan_workspace_size.restype = _sz
_SCAN_ARGS = [_P] * 12 + [_i32, _i64, _i32, _i32, _i32, _i32, _i32, _P, _sz, _P]
lib.ssdq_chunk_scan.argtypes = _SCAN_ARGS
lib.ssdq_chunk_scan.restype = ctypes.c_int
lib.ssdq_chunk_scan_stage.argtypes = [_i32] + _SCAN_ARGS
lib.ssdq_chunk_scan_stage.restype = ctypes.c_int
lib.ssdq_state_update.argtypes = [_P] * 11 + [_i32, _i32, _i32, _i32, _i32, _P]
lib.ssdq_state_update.restype = ctypes.c_int
lib.ssdq_state_update_f16.argtypes = [_P] * 11 + [_i32, _i32, _i32, _i32, _i32, _P]
lib.ssdq_state_update_f16.restype = ctypes.c_int
lib.ssdq_frontend.argtypes = [_P, _P, _P, _i32] + [_P] * 9 + [_i32, ctypes.c_int64, _i32, _i32, _i32, _i32, _P]
lib.ssdq_frontend.restype = ctypes.c_int
lib.ssdq_frontend_step.argtypes = [_P, _P, _P, _P, _i32] + [_P] * 9 + [_i32] * 5 + [_P]
lib.ssdq_frontend_step.restype = ctypes.c_int
lib.ssdq_state_update_i8.argtypes = [_P] * 12 + [_i32, _i32, _i32, _i32, _i32, _P]
lib.ssdq_state_update_i8.restype = ctypes.c_int
lib.ssdq_chunk_scan_corrected.argtypes = [_P] * 13 + [_i32, _i64, _i32, _i32, _i32, _i32, _i32, _P, _sz, _P]
lib.ssdq_chunk_scan_per_state.argtypes = [_P] * 13 + [_i32, _i64, _i32, _i32, _i32, _i32, _i32, _P, _sz, _P]
lib.ssdq_chunk_scan_per_state.restype = ctypes.c_int
lib.ssdq_chunk_scan_scaled.argtypes = [_P] * 13 + [_i32, _i64, _i32, _i32, _i32, _i32, _i32, ctypes.c_uint32, _P, _sz,
                                                  _P]
lib.ssdq_chunk_scan_scaled.restype = ctypes.c_int
lib.ssdq_state_update_scaled.argtypes = [_i32] + [_P] * 13 + [_i32, _i32, _i32, _i32, _i32, ctypes.c_uint32, _P]
lib.ssdq_state_update_scaled.restype = ctypes.c_int
lib.ssdq_state_update_per_state.argtypes = [_i32] + [_P] * 13 + [_i32, _i32, _i32, _i32, _i32, _P]
lib.ssdq_state_update_per_state.restype = ctypes.c_int
lib.ssdq_quantize_per_channel.argtypes = [_P, _P, _P, _i64, _i32, _i32, _P]
lib.ssdq_quantize_per_channel.restype = ctypes.c_int
lib.ssdq_chunk_scan_corrected.restype = ctypes.c_int
lib.ssdq_state_update_corrected.argtypes = [_i32] + [_P] * 13 + [_i32, _i32, _i32, _i32, _i32, _P]
lib.ssdq_state_update_corrected.restype = ctypes.c_int
STATE_F32, STATE_F16, STATE_I8 = 0, 1, 2
lib.ssdq_chunk_scan_noalloc.argtypes = [_P] * 12 + [_i32, _i64, _i32, _i32, _i32, _i32, _i32, _P]
lib.ssdq_chunk_scan_noalloc.restype = ctypes.c_int
lib.ssdq_chunk_scan_noalloc_scratch_size.argtypes = [_i32, _i64, _i32, _i32, _i32, _i32]
lib.ssdq_chunk_scan_noalloc_scratch_size.restype = _sz
lib.ssdq_chunk_scan_state_fused.argtypes = [_i32, _i32]
lib.ssdq_chunk_scan_state_fused.restype = _i32
lib.ssdq_chunk_scan_plan.argtypes = [_i32, _i32, ctypes.c_uint32]
lib.ssdq_chunk_scan_plan.restype = _i32


# scale layouts of ssdq_chunk_scan_scaled / ssdq_state_update_scaled (bit flags)
SCALES_BC_PER_STATE = 1   # B_scale, C_scale (ngroups, dstate)
SCALES_X_PER_CHANNEL = 2  # x_scale (nheads, headdim)


class SSDQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def chunk_scan_state_fused(batch: int, nheads: int) -> bool:
    """True when, on the current device, stage 0 of the chunk scan also carries the state across
    chunks (stage 1 then does nothing and the chunk states are not written)."""
    return bool(lib.ssdq_chunk_scan_state_fused(batch, nheads))


def chunk_scan_plan(batch: int, nheads: int, scale_layout: int = 0) -> int:
    """The form of stage 0 on the current device: 0 three kernels, 8 or 4 the folded state kernel
    in blocks of that many waves (ssdq_chunk_scan_plan)."""
    return int(lib.ssdq_chunk_scan_plan(batch, nheads, scale_layout))


def status_string(status: int) -> str:
    return lib.ssdq_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != SSDQ_SUCCESS:
        raise SSDQError(status, where)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor | None, name: str, dtype: torch.dtype, shape: tuple | None, device, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ---------------------------------------------------------------------------------------------
# quantize


class QuantizeCall:
    """A validated quantize call with its arguments marshalled once (for launch loops)."""

    def __init__(self, x: torch.Tensor, scale: torch.Tensor, out: torch.Tensor | None = None):
        if x.dim() < 2:
            raise ValueError("x must have at least 2 dimensions (..., nscale, inner)")
        nscale, inner = x.shape[-2], x.shape[-1]
        _need(x, "x", torch.float16, None, None)
        _need(scale, "scale", torch.float32, (nscale,), x.device)
        if out is None:
            out = torch.empty(x.shape, dtype=torch.int8, device=x.device)
        _need(out, "out", torch.int8, tuple(x.shape), x.device)
        rows = x.numel() // (nscale * inner) if x.numel() else 0
        self.out = out
        self.device = x.device
        self._args = (_ptr(x), _ptr(out), _ptr(scale), rows, nscale, inner)
        self._keep = (x, scale, out)

    def run(self) -> torch.Tensor:
        _check(lib.ssdq_quantize(*self._args, _stream(self.device)), "ssdq_quantize")
        return self.out


class QuantizeBatch:
    """Several quantize calls (e.g. x, B and C of one step) as one ssdq_quantize_batch call."""

    def __init__(self, calls: list[QuantizeCall]):
        if not 1 <= len(calls) <= QUANTIZE_MAX_JOBS:
            raise ValueError(f"a batch holds 1 to {QUANTIZE_MAX_JOBS} quantize calls")
        devices = {c.device for c in calls}
        if len(devices) != 1:
            raise ValueError("every tensor of a batch must be on one device")
        self.device = calls[0].device
        self.calls = calls
        self._jobs = (QuantizeJob * len(calls))(*[QuantizeJob(*c._args) for c in calls])

    def run(self) -> list[torch.Tensor]:
        _check(lib.ssdq_quantize_batch(self._jobs, len(self.calls), _stream(self.device)), "ssdq_quantize_batch")
        return [c.out for c in self.calls]


def quantize_batch(pairs, outs=None) -> list[torch.Tensor]:
    """INT8 codes of several fp16 tensors in one launch; pairs holds (x, scale) per tensor and
    outs (optional) the output tensors.  Each result equals quantize(x, scale)."""
    outs = outs if outs is not None else [None] * len(pairs)
    return QuantizeBatch([QuantizeCall(x, s, o) for (x, s), o in zip(pairs, outs)]).run()


def quantize(x: torch.Tensor, scale: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """INT8 codes of an fp16 tensor (..., S, I) with one fp32 scale per index of the
    second-to-last axis (heads for x, groups for B and C), or, with a 2-D scale (S, I), one per
    (s, i) (B and C with a scale per (group, state), x with one per (head, channel):
    ssdq_quantize_per_channel)."""
    if scale.dim() == 2:
        if x.dim() < 2:
            raise ValueError("x must have at least 2 dimensions (..., nscale, inner)")
        nscale, inner = x.shape[-2], x.shape[-1]
        _need(x, "x", torch.float16, None, None)
        _need(scale, "scale", torch.float32, (nscale, inner), x.device)
        if out is None:
            out = torch.empty(x.shape, dtype=torch.int8, device=x.device)
        _need(out, "out", torch.int8, tuple(x.shape), x.device)
        rows = x.numel() // (nscale * inner) if x.numel() else 0
        _check(lib.ssdq_quantize_per_channel(_ptr(x), _ptr(out), _ptr(scale), rows, nscale, inner, _stream(x.device)),
               "ssdq_quantize_per_channel")
        return out
    return QuantizeCall(x, scale, out).run()


# ---------------------------------------------------------------------------------------------
# prefill


def chunk_scan_workspace_size(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int, chunk: int) -> int:
    return int(lib.ssdq_chunk_scan_workspace_size(batch, seqlen, nheads, headdim, dstate, chunk))


def workspace_layout(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int, chunk: int) -> dict:
    """Offsets (bytes) and shapes of the documented workspace regions (see include/ssdq.h)."""
    r256 = lambda v: (v + 255) // 256 * 256
    nc = -(-seqlen // chunk)
    acs = r256(4 * batch * nheads * nc * chunk)
    st = 4 * batch * nc * nheads * headdim * dstate
    hp = r256(2 * batch * nc * nheads * headdim * dstate)
    return dict(nchunks=nc,
                acs=(0, "float32", (batch, nheads, nc, chunk)),
                dtc=(acs, "float32", (batch, nheads, nc, chunk)),
                states=(2 * acs, "float32", (batch, nc, nheads, headdim, dstate)),
                hprev=(2 * acs + st, "int8", (batch, nc, nheads, 2, headdim, dstate)),
                hscale=(2 * acs + st + hp, "float32", (batch, nc, nheads, headdim)))


class ScanBuffers:
    """Validated arguments of one prefill call, reusable across calls (no allocation per call)."""

    def __init__(self, x, x_scale, B, B_scale, C, C_scale, dt, A, D=None, h0=None, chunk=256, y=None,
                 h_final=None, workspace=None, want_final_state=True, y_corr=None):
        if x.dim() != 4 or B.dim() != 4:
            raise ValueError("x must be (batch, seqlen, nheads, headdim) and B, C (batch, seqlen, ngroups, dstate)")
        b, L, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        dev = x.device
        _need(x, "x", torch.int8, (b, L, H, P), dev)
        self.x_per_channel = x_scale.dim() == 2
        _need(x_scale, "x_scale", torch.float32, (H, P) if self.x_per_channel else (H,), dev)
        _need(B, "B", torch.int8, (b, L, G, N), dev)
        self.per_state = B_scale.dim() == 2
        self.scale_layout = (SCALES_BC_PER_STATE if self.per_state else 0) | (
            SCALES_X_PER_CHANNEL if self.x_per_channel else 0)
        sshape = (G, N) if self.per_state else (G,)
        _need(B_scale, "B_scale", torch.float32, sshape, dev)
        _need(C, "C", torch.int8, (b, L, G, N), dev)
        _need(C_scale, "C_scale", torch.float32, sshape, dev)
        _need(dt, "dt", torch.float32, (b, L, H), dev)
        _need(A, "A", torch.float32, (H,), dev)
        _need(D, "D", torch.float32, (H,), dev, optional=True)
        _need(h0, "h0", torch.float32, (b, H, P, N), dev, optional=True)
        _need(y_corr, "y_corr", torch.float32, (H, P), dev, optional=True)
        if y is None:
            y = torch.empty((b, L, H, P), dtype=torch.float16, device=dev)
        _need(y, "y", torch.float16, (b, L, H, P), dev)
        if h_final is None and want_final_state:
            h_final = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
        _need(h_final, "h_final", torch.float32, (b, H, P, N), dev, optional=True)
        ws = chunk_scan_workspace_size(b, L, H, P, N, chunk)
        if ws == 0:
            raise SSDQError(SSDQ_ERROR_UNSUPPORTED, "ssdq_chunk_scan_workspace_size")
        if workspace is None:
            workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
        _need(workspace, "workspace", torch.uint8, None, dev)
        self.tensors = (x, x_scale, B, B_scale, C, C_scale, dt, A, D, h0, y, h_final)
        self.y_corr = y_corr
        self.dims = (b, L, H, P, N, G, chunk)
        self.workspace = workspace
        self.device = dev
        self.y, self.h_final = y, h_final
        self._args = [_ptr(t) for t in self.tensors] + list(self.dims) + [
            _ptr(workspace), workspace.numel()]

    def run(self) -> None:
        """The whole scan: ssdq_chunk_scan; ssdq_chunk_scan_corrected with an output correction;
        ssdq_chunk_scan_per_state with B, C scales per (group, state) only; ssdq_chunk_scan_scaled
        with x scales per (head, channel)."""
        a = self._args
        if self.x_per_channel:
            _check(lib.ssdq_chunk_scan_scaled(*a[:9], _ptr(self.y_corr), *a[9:-2], self.scale_layout, *a[-2:],
                                              _stream(self.device)), "ssdq_chunk_scan_scaled")
        elif self.per_state:
            _check(lib.ssdq_chunk_scan_per_state(*a[:9], _ptr(self.y_corr), *a[9:], _stream(self.device)),
                   "ssdq_chunk_scan_per_state")
        elif self.y_corr is not None:
            _check(lib.ssdq_chunk_scan_corrected(*a[:9], _ptr(self.y_corr), *a[9:], _stream(self.device)),
                   "ssdq_chunk_scan_corrected")
        else:
            _check(lib.ssdq_chunk_scan(*self._args, _stream(self.device)), "ssdq_chunk_scan")

    def run_stage(self, stage: int) -> None:
        if self.y_corr is not None or self.scale_layout:
            raise ValueError("the stage-level calls take neither an output correction nor finer scales; use run()")
        _check(lib.ssdq_chunk_scan_stage(stage, *self._args, _stream(self.device)), "ssdq_chunk_scan_stage")

    def workspace_views(self) -> dict:
        """Typed views of the workspace regions (for inspecting stage results)."""
        b, L, H, P, N, G, Q = self.dims
        lay = workspace_layout(b, L, H, P, N, Q)
        out = {}
        for key in ("acs", "dtc", "states", "hprev", "hscale"):
            off, dtype, shape = lay[key]
            dt = getattr(torch, dtype)
            n = 1
            for d in shape:
                n *= d
            nbytes = n * torch.empty((), dtype=dt).element_size()
            out[key] = self.workspace[off:off + nbytes].view(dt).view(shape)
        return out


def chunk_scan(x, x_scale, B, B_scale, C, C_scale, dt, A, D=None, h0=None, chunk=256, y=None, h_final=None,
               workspace=None, want_final_state=True, y_corr=None):
    """Prefill over INT8 inputs; returns (y fp16 (b,L,H,P), h_final fp32 (b,H,P,N) or None).  y_corr
    (H, P) fp32, if given, is the output correction added to every y (ssdq_chunk_scan_corrected)."""
    buf = ScanBuffers(x, x_scale, B, B_scale, C, C_scale, dt, A, D, h0, chunk, y, h_final, workspace,
                      want_final_state, y_corr)
    buf.run()
    return buf.y, buf.h_final


def chunk_scan_noalloc_scratch_size(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int,
                                    chunk: int) -> int:
    return int(lib.ssdq_chunk_scan_noalloc_scratch_size(batch, seqlen, nheads, headdim, dstate, chunk))


def chunk_scan_noalloc(x, x_scale, B, B_scale, C, C_scale, dt, A, D=None, h0=None, chunk=256, y=None,
                       h_final=None):
    """Prefill through ssdq_chunk_scan_noalloc: the library's static device scratch instead of a
    workspace (the call itself allocates nothing; y and h_final are allocated here unless given).
    Returns (y, h_final)."""
    b, L, H, P = x.shape
    N = B.shape[3]
    dev = x.device
    if y is None:
        y = torch.empty((b, L, H, P), dtype=torch.float16, device=dev)
    if h_final is None:
        h_final = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
    # the same argument checks as ScanBuffers, with no workspace
    G = B.shape[2]
    for t, name, dtype, shape, opt in ((x, "x", torch.int8, (b, L, H, P), False),
                                      (x_scale, "x_scale", torch.float32, (H,), False),
                                      (B, "B", torch.int8, (b, L, G, N), False),
                                      (B_scale, "B_scale", torch.float32, (G,), False),
                                      (C, "C", torch.int8, (b, L, G, N), False),
                                      (C_scale, "C_scale", torch.float32, (G,), False),
                                      (dt, "dt", torch.float32, (b, L, H), False), (A, "A", torch.float32, (H,), False),
                                      (D, "D", torch.float32, (H,), True), (h0, "h0", torch.float32, (b, H, P, N), True),
                                      (y, "y", torch.float16, (b, L, H, P), False),
                                      (h_final, "h_final", torch.float32, (b, H, P, N), False)):
        _need(t, name, dtype, shape, dev, optional=opt)
    args = [_ptr(t) for t in (x, x_scale, B, B_scale, C, C_scale, dt, A, D, h0, y, h_final)]
    _check(lib.ssdq_chunk_scan_noalloc(*args, b, L, H, P, N, G, chunk, _stream(dev)), "ssdq_chunk_scan_noalloc")
    return y, h_final


# ---------------------------------------------------------------------------------------------
# decode


def frontend(xbc, conv_w, conv_b, x_scale, B_scale, C_scale, dt_raw, dt_bias, nheads: int, headdim: int,
             ngroups: int, dstate: int, out=None):
    """The block's front end fused with the quantizer (ssdq_frontend): xbc (b,L,H*P+2*G*N) fp16
    -> codes x (b,L,H,P), B, C (b,L,G,N) int8 and dt (b,L,H) fp32 = softplus(dt_raw + dt_bias).
    Returns (x, B, C, dt); `out` may give those four tensors."""
    if xbc.dim() != 3:
        raise ValueError("xbc must be (batch, seqlen, channels)")
    b, L, ch = xbc.shape
    H, P, G, N = nheads, headdim, ngroups, dstate
    dev = xbc.device
    _need(xbc, "xbc", torch.float16, (b, L, H * P + 2 * G * N), dev)
    _need(conv_w, "conv_w", torch.float32, (ch, 4), dev)
    _need(conv_b, "conv_b", torch.float32, (ch,), dev, optional=True)
    _need(x_scale, "x_scale", torch.float32, (H,), dev)
    _need(B_scale, "B_scale", torch.float32, (G,), dev)
    _need(C_scale, "C_scale", torch.float32, (G,), dev)
    _need(dt_raw, "dt_raw", torch.float32, (b, L, H), dev)
    _need(dt_bias, "dt_bias", torch.float32, (H,), dev, optional=True)
    if out is None:
        out = (torch.empty((b, L, H, P), dtype=torch.int8, device=dev),
               torch.empty((b, L, G, N), dtype=torch.int8, device=dev),
               torch.empty((b, L, G, N), dtype=torch.int8, device=dev),
               torch.empty((b, L, H), dtype=torch.float32, device=dev))
    x, B, C, dt = out
    _need(x, "x", torch.int8, (b, L, H, P), dev)
    _need(B, "B", torch.int8, (b, L, G, N), dev)
    _need(C, "C", torch.int8, (b, L, G, N), dev)
    _need(dt, "dt", torch.float32, (b, L, H), dev)
    _check(lib.ssdq_frontend(_ptr(xbc), _ptr(conv_w), _ptr(conv_b), 4, _ptr(x_scale), _ptr(B_scale),
                             _ptr(C_scale), _ptr(dt_raw), _ptr(dt_bias), _ptr(x), _ptr(B), _ptr(C), _ptr(dt), b, L,
                             H, P, N, G, _stream(dev)), "ssdq_frontend")
    return x, B, C, dt


def frontend_step(conv_state, xbc, conv_w, conv_b, x_scale, B_scale, C_scale, dt_raw, dt_bias, nheads: int,
                  headdim: int, ngroups: int, dstate: int, out=None):
    """One decode token of the front end (ssdq_frontend_step): conv_state (b,3,channels) fp16 is
    shifted in place; xbc (b,channels) fp16 -> codes x (b,H,P), B, C (b,G,N) and dt (b,H).
    Returns (x, B, C, dt); `out` may give those four tensors."""
    b, ch = xbc.shape
    H, P, G, N = nheads, headdim, ngroups, dstate
    dev = xbc.device
    _need(xbc, "xbc", torch.float16, (b, H * P + 2 * G * N), dev)
    _need(conv_state, "conv_state", torch.float16, (b, 3, ch), dev)
    _need(conv_w, "conv_w", torch.float32, (ch, 4), dev)
    _need(conv_b, "conv_b", torch.float32, (ch,), dev, optional=True)
    _need(x_scale, "x_scale", torch.float32, (H,), dev)
    _need(B_scale, "B_scale", torch.float32, (G,), dev)
    _need(C_scale, "C_scale", torch.float32, (G,), dev)
    _need(dt_raw, "dt_raw", torch.float32, (b, H), dev)
    _need(dt_bias, "dt_bias", torch.float32, (H,), dev, optional=True)
    if out is None:
        out = (torch.empty((b, H, P), dtype=torch.int8, device=dev),
               torch.empty((b, G, N), dtype=torch.int8, device=dev),
               torch.empty((b, G, N), dtype=torch.int8, device=dev),
               torch.empty((b, H), dtype=torch.float32, device=dev))
    x, B, C, dt = out
    _need(x, "x", torch.int8, (b, H, P), dev)
    _need(B, "B", torch.int8, (b, G, N), dev)
    _need(C, "C", torch.int8, (b, G, N), dev)
    _need(dt, "dt", torch.float32, (b, H), dev)
    _check(lib.ssdq_frontend_step(_ptr(conv_state), _ptr(xbc), _ptr(conv_w), _ptr(conv_b), 4, _ptr(x_scale),
                                  _ptr(B_scale), _ptr(C_scale), _ptr(dt_raw), _ptr(dt_bias), _ptr(x), _ptr(B),
                                  _ptr(C), _ptr(dt), b, H, P, N, G, _stream(dev)), "ssdq_frontend_step")
    return x, B, C, dt


def state_update(state, x, x_scale, B, B_scale, C, C_scale, dt, A, D=None, y=None, state_scale=None,
                 y_corr=None) -> torch.Tensor:
    """One decode step; `state` (b,H,P,N) is updated in place; returns y fp16 (b,H,P).  An fp32
    state runs ssdq_state_update, a binary16 (torch.float16) state ssdq_state_update_f16, and an
    int8 state (codes, with its row scales `state_scale` (b,H,P) float32, also updated in place)
    ssdq_state_update_i8; with y_corr (H, P) fp32 the step runs ssdq_state_update_corrected and
    y also receives that output correction; with B and C scales per (group, state) (G, N) it runs
    ssdq_state_update_per_state (y_corr optional); with x scales per (head, channel) (H, P) it
    runs ssdq_state_update_scaled (with either B, C layout; y_corr optional)."""
    if state.dim() != 4:
        raise ValueError("state must be (batch, nheads, headdim, dstate)")
    b, H, P, N = state.shape
    G = B.shape[1] if B.dim() == 3 else -1
    dev = state.device
    kind = {torch.float16: "f16", torch.int8: "i8"}.get(state.dtype, "f32")
    _need(state, "state", {"f16": torch.float16, "i8": torch.int8}.get(kind, torch.float32), (b, H, P, N), dev)
    if kind == "i8":
        _need(state_scale, "state_scale", torch.float32, (b, H, P), dev)
    elif state_scale is not None:
        raise ValueError("state_scale goes with an int8 state only")
    per_state = B_scale.dim() == 2
    x_per_channel = x_scale.dim() == 2
    sshape = (G, N) if per_state else (G,)
    _need(x, "x", torch.int8, (b, H, P), dev)
    _need(x_scale, "x_scale", torch.float32, (H, P) if x_per_channel else (H,), dev)
    _need(B, "B", torch.int8, (b, G, N), dev)
    _need(B_scale, "B_scale", torch.float32, sshape, dev)
    _need(C, "C", torch.int8, (b, G, N), dev)
    _need(C_scale, "C_scale", torch.float32, sshape, dev)
    _need(dt, "dt", torch.float32, (b, H), dev)
    _need(A, "A", torch.float32, (H,), dev)
    _need(D, "D", torch.float32, (H,), dev, optional=True)
    _need(y_corr, "y_corr", torch.float32, (H, P), dev, optional=True)
    if y is None:
        y = torch.empty((b, H, P), dtype=torch.float16, device=dev)
    _need(y, "y", torch.float16, (b, H, P), dev)
    if x_per_channel:
        fmt = {"f32": STATE_F32, "f16": STATE_F16, "i8": STATE_I8}[kind]
        layout = SCALES_X_PER_CHANNEL | (SCALES_BC_PER_STATE if per_state else 0)
        _check(lib.ssdq_state_update_scaled(fmt, _ptr(state), _ptr(state_scale), _ptr(x), _ptr(x_scale), _ptr(B),
                                            _ptr(B_scale), _ptr(C), _ptr(C_scale), _ptr(dt), _ptr(A), _ptr(D),
                                            _ptr(y_corr), _ptr(y), b, H, P, N, G, layout, _stream(dev)),
               "ssdq_state_update_scaled")
        return y
    if per_state:
        fmt = {"f32": STATE_F32, "f16": STATE_F16, "i8": STATE_I8}[kind]
        _check(lib.ssdq_state_update_per_state(fmt, _ptr(state), _ptr(state_scale), _ptr(x), _ptr(x_scale), _ptr(B),
                                               _ptr(B_scale), _ptr(C), _ptr(C_scale), _ptr(dt), _ptr(A), _ptr(D),
                                               _ptr(y_corr), _ptr(y), b, H, P, N, G, _stream(dev)),
               "ssdq_state_update_per_state")
        return y
    if y_corr is not None:
        fmt = {"f32": STATE_F32, "f16": STATE_F16, "i8": STATE_I8}[kind]
        _check(lib.ssdq_state_update_corrected(fmt, _ptr(state), _ptr(state_scale), _ptr(x), _ptr(x_scale), _ptr(B),
                                               _ptr(B_scale), _ptr(C), _ptr(C_scale), _ptr(dt), _ptr(A), _ptr(D),
                                               _ptr(y_corr), _ptr(y), b, H, P, N, G, _stream(dev)),
               "ssdq_state_update_corrected")
        return y
    rest = (_ptr(x), _ptr(x_scale), _ptr(B), _ptr(B_scale), _ptr(C), _ptr(C_scale), _ptr(dt), _ptr(A), _ptr(D),
            _ptr(y), b, H, P, N, G, _stream(dev))
    if kind == "i8":
        _check(lib.ssdq_state_update_i8(_ptr(state), _ptr(state_scale), *rest), "ssdq_state_update_i8")
    elif kind == "f16":
        _check(lib.ssdq_state_update_f16(_ptr(state), *rest), "ssdq_state_update_f16")
    else:
        _check(lib.ssdq_state_update(_ptr(state), *rest), "ssdq_state_update")
    return y
