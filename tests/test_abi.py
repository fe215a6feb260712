"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any launch.

Pointers passed here are fake (aligned or misaligned integers); every call is
made with at least one invalid argument, so validation returns before the
library touches the HIP runtime or any memory.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssdq.h")
LIB = os.path.join(ROOT, "quantized_selective_state_amd", "libssdq.so")

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3
A16 = 0x100000  # a fake, 16-byte aligned address (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libssdq.so not built")
    lib = ctypes.CDLL(LIB)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    scan = [P] * 12 + [i32, i64, i32, i32, i32, i32, i32, P, sz, P]
    lib.ssdq_chunk_scan.argtypes = scan
    lib.ssdq_chunk_scan_stage.argtypes = [i32] + scan
    lib.ssdq_quantize.argtypes = [P, P, P, i64, i32, i32, P]
    lib.ssdq_chunk_scan_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32]
    lib.ssdq_chunk_scan_workspace_size.restype = sz
    lib.ssdq_state_update.argtypes = [P] * 11 + [i32] * 5 + [P]
    lib.ssdq_state_update_f16.argtypes = [P] * 11 + [i32] * 5 + [P]
    lib.ssdq_state_update_i8.argtypes = [P] * 12 + [i32] * 5 + [P]
    lib.ssdq_frontend_step.argtypes = [P, P, P, P, i32] + [P] * 9 + [i32] * 5 + [P]
    lib.ssdq_frontend.argtypes = [P, P, P, i32] + [P] * 9 + [i32, i64, i32, i32, i32, i32, P]
    lib.ssdq_status_string.argtypes = [ctypes.c_int]
    lib.ssdq_status_string.restype = ctypes.c_char_p
    return lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssdq_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("ssdq_quantize", "ssdq_chunk_scan", "ssdq_state_update"):
        assert n in names


def test_every_declared_function_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert lib.ssdq_status_string(0) == b"SSDQ_SUCCESS"
    assert lib.ssdq_status_string(3) == b"SSDQ_ERROR_WORKSPACE_TOO_SMALL"
    assert lib.ssdq_status_string(99) == b"SSDQ_UNKNOWN_STATUS"


def _ws(b, L, H, P, N, Q):
    r = lambda v: (v + 255) // 256 * 256
    nc = -(-L // Q)
    return (2 * r(4 * b * H * nc * Q) + 4 * b * nc * H * P * N + r(2 * b * nc * H * P * N) + r(4 * b * nc * H * P))


def test_workspace_size(lib):
    # Acs fp32 + chunk-ordered dt fp32 + chunk states fp32 + carried-state limbs (2 x int8) + row
    # scales fp32, 256-byte aligned regions
    assert lib.ssdq_chunk_scan_workspace_size(4, 2048, 64, 64, 128, 256) == _ws(4, 2048, 64, 64, 128, 256)
    assert lib.ssdq_chunk_scan_workspace_size(1, 250, 2, 16, 16, 64) == _ws(1, 250, 2, 16, 16, 64)
    assert _ws(1, 250, 2, 16, 16, 64) == 2 * 2048 + 4 * 4 * 2 * 16 * 16 + 2 * 4 * 2 * 16 * 16 + 512
    assert lib.ssdq_chunk_scan_workspace_size(1, 256, 4, 16, 16, 48) == 0     # unsupported chunk
    assert lib.ssdq_chunk_scan_workspace_size(0, 256, 4, 16, 16, 64) == 0


def _scan(lib, **kw):
    args = dict(x=A16, xs=A16, B=A16, Bs=A16, C=A16, Cs=A16, dt=A16, A=A16, D=None, h0=None, y=A16, hf=None,
                b=1, L=256, H=4, P=16, N=16, G=1, Q=64, ws=A16, wsb=1 << 30, stream=None, stage=None)
    args.update(kw)
    vals = [args[k] for k in ("x", "xs", "B", "Bs", "C", "Cs", "dt", "A", "D", "h0", "y", "hf", "b", "L", "H",
                              "P", "N", "G", "Q", "ws", "wsb", "stream")]
    if args["stage"] is None:
        return lib.ssdq_chunk_scan(*vals)
    return lib.ssdq_chunk_scan_stage(args["stage"], *vals)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID),
    (dict(y=None), INVALID),
    (dict(ws=None), INVALID),
    (dict(dt=A16 + 4), INVALID),          # misaligned
    (dict(h0=A16 + 8), INVALID),
    (dict(b=0), INVALID),
    (dict(L=0), INVALID),
    (dict(Q=0), INVALID),
    (dict(H=6, G=4), INVALID),            # H % G != 0
    (dict(P=24), UNSUPPORTED),
    (dict(P=128), UNSUPPORTED),
    (dict(N=8), UNSUPPORTED),
    (dict(N=256), UNSUPPORTED),
    (dict(Q=32), UNSUPPORTED),
    (dict(Q=100), UNSUPPORTED),
    (dict(H=1 << 17, G=1, P=64, N=16, Q=256), UNSUPPORTED),        # a chunk of x: 2^31 bytes
    (dict(H=1 << 16, G=1, P=64, N=16, Q=256), UNSUPPORTED),        # a chunk of fp16 y: 2^31 bytes
    (dict(H=1 << 16, G=1 << 16, P=16, N=128, Q=256), UNSUPPORTED),  # a chunk of B, C: 2^31 bytes
    (dict(wsb=100), WS_SMALL),
    (dict(stage=3, wsb=100), INVALID),
    (dict(stage=-1), INVALID),
    (dict(stage=2, wsb=100), WS_SMALL),
])
def test_chunk_scan_validation(lib, kw, status):
    assert _scan(lib, **kw) == status


@pytest.mark.parametrize("args,status", [
    ((None, A16, A16, 10, 4, 16), INVALID),
    ((A16, A16, A16, -1, 4, 16), INVALID),
    ((A16, A16, A16, 10, 0, 16), INVALID),
    ((A16, A16, A16, 10, 4, 0), INVALID),
    ((A16 + 2, A16, A16, 10, 4, 16), INVALID),
    ((None, None, None, 0, 4, 16), OK),    # rows == 0: nothing to do
])
def test_quantize_validation(lib, args, status):
    assert lib.ssdq_quantize(*args, None) == status


class Job(ctypes.Structure):
    _fields_ = [("x_f16", ctypes.c_void_p), ("q", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("nscale", ctypes.c_int32), ("inner", ctypes.c_int32)]


def test_quantize_job_layout():
    # the C struct: three pointers, an int64 and two int32 (no padding)
    assert ctypes.sizeof(Job) == 40
    assert "SSDQ_QUANTIZE_MAX_JOBS 8" in open(HEADER).read()


@pytest.mark.parametrize("jobs,count,status", [
    ([], 0, INVALID),                                             # count below 1
    ([(A16, A16, A16, 10, 4, 16)] * 9, 9, INVALID),               # count above the maximum
    ([(A16, A16, A16, 10, 4, 16), (A16, A16, A16, -1, 4, 16)], 2, INVALID),
    ([(A16, A16, A16, 10, 4, 16), (A16, A16, A16, 10, 0, 16)], 2, INVALID),
    ([(A16, A16, A16, 10, 4, 0)], 1, INVALID),
    ([(A16, A16 + 1, A16, 10, 4, 16)], 1, INVALID),               # misaligned output
    ([(A16, A16, None, 10, 4, 16)], 1, INVALID),                  # missing scales
    ([(None, None, None, 0, 4, 16), (None, None, None, 0, 2, 8)], 2, OK),   # nothing to do
])
def test_quantize_batch_validation(lib, jobs, count, status):
    lib.ssdq_quantize_batch.argtypes = [ctypes.POINTER(Job), ctypes.c_int32, ctypes.c_void_p]
    arr = (Job * max(len(jobs), 1))(*[Job(*j) for j in jobs])
    assert lib.ssdq_quantize_batch(arr, count, None) == status


def test_quantize_batch_rejects_null_jobs(lib):
    lib.ssdq_quantize_batch.argtypes = [ctypes.POINTER(Job), ctypes.c_int32, ctypes.c_void_p]
    assert lib.ssdq_quantize_batch(None, 1, None) == INVALID


def _upd(lib, kind="f32", **kw):
    a = dict(state=A16, scale=A16, x=A16, xs=A16, B=A16, Bs=A16, C=A16, Cs=A16, dt=A16, A=A16, D=None, y=A16,
             b=2, H=8, P=64, N=128, G=2)
    a.update(kw)
    rest = [a[k] for k in ("x", "xs", "B", "Bs", "C", "Cs", "dt", "A", "D", "y", "b", "H", "P", "N", "G")]
    if kind == "i8":
        return lib.ssdq_state_update_i8(a["state"], a["scale"], *rest, None)
    call = lib.ssdq_state_update_f16 if kind == "f16" else lib.ssdq_state_update
    return call(a["state"], *rest, None)


@pytest.mark.parametrize("kw,status", [
    (dict(state=None), INVALID),
    (dict(y=A16 + 1), INVALID),
    (dict(b=0), INVALID),
    (dict(H=8, G=3), INVALID),
    (dict(N=96), UNSUPPORTED),
    (dict(P=128), UNSUPPORTED),
])
@pytest.mark.parametrize("kind", ["f32", "f16", "i8"])   # fp32, binary16-cached and 8-bit-cached state
def test_state_update_validation(lib, kw, status, kind):
    assert _upd(lib, kind=kind, **kw) == status


@pytest.mark.parametrize("scale", [None, A16 + 4])
def test_state_update_i8_needs_an_aligned_scale(lib, scale):
    assert _upd(lib, kind="i8", scale=scale) == INVALID


def _fe(lib, **kw):
    a = dict(xbc=A16, w=A16, bias=None, dconv=4, xs=A16, Bs=A16, Cs=A16, raw=A16, dtb=None, x=A16, B=A16, C=A16,
             dt=A16, b=2, L=100, H=8, P=64, N=128, G=2)
    a.update(kw)
    return lib.ssdq_frontend(*[a[k] for k in ("xbc", "w", "bias", "dconv", "xs", "Bs", "Cs", "raw", "dtb", "x", "B",
                                              "C", "dt", "b", "L", "H", "P", "N", "G")], None)


@pytest.mark.parametrize("kw,status", [
    (dict(xbc=None), INVALID),
    (dict(dt=A16 + 4), INVALID),
    (dict(bias=A16 + 8), INVALID),
    (dict(b=0), INVALID),
    (dict(L=-1), INVALID),
    (dict(H=8, G=3), INVALID),
    (dict(dconv=3), UNSUPPORTED),
    (dict(P=20), UNSUPPORTED),
    (dict(N=12), UNSUPPORTED),
    (dict(b=65536, L=(1 << 19)), UNSUPPORTED),   # 2^16 batches * 4 channel blocks * 2^15 strips
    (dict(L=0, xbc=None, x=None), OK),
])
def test_frontend_validation(lib, kw, status):
    assert _fe(lib, **kw) == status


def _fes(lib, **kw):
    a = dict(st=A16, xbc=A16, w=A16, bias=None, dconv=4, xs=A16, Bs=A16, Cs=A16, raw=A16, dtb=None, x=A16, B=A16,
             C=A16, dt=A16, b=2, H=8, P=64, N=128, G=2)
    a.update(kw)
    return lib.ssdq_frontend_step(*[a[k] for k in ("st", "xbc", "w", "bias", "dconv", "xs", "Bs", "Cs", "raw", "dtb",
                                                   "x", "B", "C", "dt", "b", "H", "P", "N", "G")], None)


@pytest.mark.parametrize("kw,status", [
    (dict(st=None), INVALID),
    (dict(st=A16 + 2), INVALID),
    (dict(b=0), INVALID),
    (dict(H=8, G=3), INVALID),
    (dict(dconv=2), UNSUPPORTED),
    (dict(P=12), UNSUPPORTED),
])
def test_frontend_step_validation(lib, kw, status):
    assert _fes(lib, **kw) == status


def test_noalloc_validates_before_touching_the_device(lib):
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.ssdq_chunk_scan_noalloc.argtypes = [P] * 12 + [i32, i64, i32, i32, i32, i32, i32, P]
    lib.ssdq_chunk_scan_noalloc_scratch_size.argtypes = [i32, i64, i32, i32, i32, i32]
    lib.ssdq_chunk_scan_noalloc_scratch_size.restype = sz
    ptrs = [A16] * 12
    # a misaligned pointer, a bad shape, an unsupported shape: rejected like ssdq_chunk_scan
    bad = list(ptrs)
    bad[0] = A16 + 1
    assert lib.ssdq_chunk_scan_noalloc(*bad, 1, 256, 4, 16, 16, 1, 64, None) == INVALID
    assert lib.ssdq_chunk_scan_noalloc(*ptrs, 1, 256, 3, 16, 16, 2, 64, None) == INVALID      # H % G
    assert lib.ssdq_chunk_scan_noalloc(*ptrs, 1, 256, 4, 24, 16, 1, 64, None) == UNSUPPORTED  # headdim
    # the 8B-shaped layer's intermediates (256 MiB of carried state) exceed the 64 MiB scratch: the
    # call says so and launches nothing, whichever plan the device would take
    need = lib.ssdq_chunk_scan_noalloc_scratch_size(8, 4096, 128, 64, 128, 256)
    assert need > 64 << 20
    assert lib.ssdq_chunk_scan_noalloc(*ptrs, 8, 4096, 128, 64, 128, 8, 256, None) == 5
    assert lib.ssdq_status_string(5) == b"SSDQ_ERROR_SCRATCH_LIMIT"
    # the compact layout without a device (three-kernel plan: the fp32 chunk states included)
    r = lambda v: (v + 255) // 256 * 256
    b, L, H, Pd, N, Q = 1, 300, 8, 32, 64, 64
    nc = -(-L // Q)
    assert lib.ssdq_chunk_scan_noalloc_scratch_size(b, L, H, Pd, N, Q) == (
        2 * r(4 * b * H * nc * Q) + r(4 * b * nc * H * Pd * N) + r(2 * b * nc * H * Pd * N) + r(4 * b * nc * H * Pd))
    assert lib.ssdq_chunk_scan_noalloc_scratch_size(0, L, H, Pd, N, Q) == 0


def test_corrected_calls_validate_on_the_host(lib):
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.ssdq_chunk_scan_corrected.argtypes = [P] * 13 + [i32, i64, i32, i32, i32, i32, i32, P, sz, P]
    lib.ssdq_state_update_corrected.argtypes = [i32] + [P] * 13 + [i32] * 5 + [P]
    ptrs = [A16] * 13
    no_corr = list(ptrs)
    no_corr[9] = None                                   # y_corr
    assert lib.ssdq_chunk_scan_corrected(*no_corr, 1, 256, 4, 16, 16, 1, 64, A16, 1 << 30, None) == INVALID
    assert lib.ssdq_chunk_scan_corrected(*ptrs, 1, 256, 4, 16, 16, 1, 64, A16, 16, None) == WS_SMALL
    assert lib.ssdq_chunk_scan_corrected(*ptrs, 1, 256, 3, 16, 16, 2, 64, A16, 1 << 30, None) == INVALID
    dec = [A16] * 13
    assert lib.ssdq_state_update_corrected(3, *dec, 2, 4, 64, 128, 2, None) == INVALID        # no such format
    bad = list(dec)
    bad[11] = None                                      # y_corr
    assert lib.ssdq_state_update_corrected(0, *bad, 2, 4, 64, 128, 2, None) == INVALID
    no_scale = list(dec)
    no_scale[1] = None                                  # state_scale, needed by the 8-bit format only
    assert lib.ssdq_state_update_corrected(2, *no_scale, 2, 4, 64, 128, 2, None) == INVALID
    assert lib.ssdq_state_update_corrected(0, *no_scale, 2, 4, 64, 96, 2, None) == UNSUPPORTED


def test_per_state_calls_validate_on_the_host(lib):
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.ssdq_chunk_scan_per_state.argtypes = [P] * 13 + [i32, i64, i32, i32, i32, i32, i32, P, sz, P]
    lib.ssdq_state_update_per_state.argtypes = [i32] + [P] * 13 + [i32] * 5 + [P]
    lib.ssdq_quantize_per_channel.argtypes = [P, P, P, i64, i32, i32, P]
    ptrs = [A16] * 13
    odd = list(ptrs)
    odd[9] = A16 + 4                                     # y_corr (optional) misaligned
    assert lib.ssdq_chunk_scan_per_state(*odd, 1, 256, 4, 16, 16, 1, 64, A16, 1 << 30, None) == INVALID
    assert lib.ssdq_chunk_scan_per_state(*ptrs, 1, 256, 4, 16, 16, 1, 64, A16, 16, None) == WS_SMALL
    assert lib.ssdq_chunk_scan_per_state(*ptrs, 1, 256, 3, 16, 16, 2, 64, A16, 1 << 30, None) == INVALID
    no_B_scale = list(ptrs)
    no_B_scale[3] = None
    assert lib.ssdq_chunk_scan_per_state(*no_B_scale, 1, 256, 4, 16, 16, 1, 64, A16, 1 << 30, None) == INVALID
    dec = [A16] * 13
    assert lib.ssdq_state_update_per_state(3, *dec, 2, 4, 64, 128, 2, None) == INVALID        # no such format
    bad = list(dec)
    bad[11] = A16 + 4                                    # y_corr misaligned
    assert lib.ssdq_state_update_per_state(0, *bad, 2, 4, 64, 128, 2, None) == INVALID
    no_scale = list(dec)
    no_scale[1] = None                                   # state_scale, needed by the 8-bit format only
    assert lib.ssdq_state_update_per_state(2, *no_scale, 2, 4, 64, 128, 2, None) == INVALID
    assert lib.ssdq_state_update_per_state(0, *no_scale, 2, 4, 64, 96, 2, None) == UNSUPPORTED
    assert lib.ssdq_quantize_per_channel(A16, A16, A16, -1, 2, 16, None) == INVALID
    assert lib.ssdq_quantize_per_channel(A16, A16, None, 4, 2, 16, None) == INVALID
    assert lib.ssdq_quantize_per_channel(A16, A16, A16, 4, 0, 16, None) == INVALID
    assert lib.ssdq_quantize_per_channel(None, None, None, 0, 2, 16, None) == 0                # nothing to do


def test_scaled_calls_validate_on_the_host(lib):
    P, i32, i64, sz, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_uint32
    lib.ssdq_chunk_scan_scaled.argtypes = [P] * 13 + [i32, i64, i32, i32, i32, i32, i32, u32, P, sz, P]
    lib.ssdq_state_update_scaled.argtypes = [i32] + [P] * 13 + [i32] * 5 + [u32, P]
    ptrs = [A16] * 13
    for layout in (4, 8, 0x80000000):                    # bits beyond the two layouts
        assert lib.ssdq_chunk_scan_scaled(*ptrs, 1, 256, 4, 16, 16, 1, 64, layout, A16, 1 << 30, None) == INVALID
    odd = list(ptrs)
    odd[9] = A16 + 4                                     # y_corr (optional) misaligned
    assert lib.ssdq_chunk_scan_scaled(*odd, 1, 256, 4, 16, 16, 1, 64, 2, A16, 1 << 30, None) == INVALID
    assert lib.ssdq_chunk_scan_scaled(*ptrs, 1, 256, 4, 16, 16, 1, 64, 3, A16, 16, None) == WS_SMALL
    assert lib.ssdq_chunk_scan_scaled(*ptrs, 1, 256, 3, 16, 16, 2, 64, 2, A16, 1 << 30, None) == INVALID
    assert lib.ssdq_chunk_scan_scaled(*ptrs, 1, 256, 4, 24, 16, 1, 64, 2, A16, 1 << 30, None) == UNSUPPORTED
    no_x_scale = list(ptrs)
    no_x_scale[1] = None
    assert lib.ssdq_chunk_scan_scaled(*no_x_scale, 1, 256, 4, 16, 16, 1, 64, 2, A16, 1 << 30, None) == INVALID
    dec = [A16] * 13
    assert lib.ssdq_state_update_scaled(3, *dec, 2, 4, 64, 128, 2, 2, None) == INVALID      # no such format
    assert lib.ssdq_state_update_scaled(0, *dec, 2, 4, 64, 128, 2, 4, None) == INVALID      # unknown layout bit
    bad = list(dec)
    bad[11] = A16 + 4                                    # y_corr misaligned
    assert lib.ssdq_state_update_scaled(0, *bad, 2, 4, 64, 128, 2, 2, None) == INVALID
    no_scale = list(dec)
    no_scale[1] = None                                   # state_scale, needed by the 8-bit format only
    assert lib.ssdq_state_update_scaled(2, *no_scale, 2, 4, 64, 128, 2, 3, None) == INVALID
    assert lib.ssdq_state_update_scaled(0, *no_scale, 2, 4, 64, 96, 2, 2, None) == UNSUPPORTED


def test_plan_query_on_the_host(lib):
    lib.ssdq_chunk_scan_plan.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32]
    lib.ssdq_chunk_scan_plan.restype = ctypes.c_int32
    assert lib.ssdq_chunk_scan_plan(0, 4, 0) == -1
    assert lib.ssdq_chunk_scan_plan(1, -4, 0) == -1
    assert lib.ssdq_chunk_scan_plan(1, 4, 4) == -1                 # unknown layout bit
    assert lib.ssdq_chunk_scan_plan(8, 128, 3) in (0, 4, 8)        # 0 where no device is visible
