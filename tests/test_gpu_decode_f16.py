"""GPU parity of ssdq_state_update_f16: the decode step with the state cached in IEEE binary16.

Against the oracle with the same caching (state rounded to binary16 after every step, y from
the update before rounding), every step: the two differ only where the fp32 update on the GPU
and the exact update fall on different sides of a binary16 rounding midpoint; such a flip moves
that element by one binary16 spacing (at most 2^-10 of its magnitude) and decays afterwards, so
the bound is a few spacings of the largest state.  Against the fp32-state recurrence, the cache
stays within one rounding per step (T * 2^-11 of the largest state on the way) plus the same
few spacings.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import Y_TOL, dev, note, threaded, to_dev

pytestmark = pytest.mark.gpu

SPACING = 2.0 ** -10   # binary16 spacing relative to a value in its binade (upper bound)
FLIPS = 4              # spacings allowed for rounding flips between the fp32 and the exact update


def _as_cache(dec):
    """The decode draw with its starting state already a binary16 value (the cache's content)."""
    dec = dict(dec)
    dec["state"] = dec["state"].astype(np.float16).astype(np.float32)
    return dec


def _gpu_decode_f16(dec, with_D=True):
    """Quantize every step's x, B, C and run the steps on a binary16 state; returns
    (y (T,b,H,P), final state as float64)."""
    import quantized_selective_state_amd as ssdq
    sx, sB, sC = to_dev(dec["x_scale"]), to_dev(dec["B_scale"]), to_dev(dec["C_scale"])
    qx = ssdq.quantize(to_dev(dec["x16"]), sx)
    qB = ssdq.quantize(to_dev(dec["B16"]), sB)
    qC = ssdq.quantize(to_dev(dec["C16"]), sC)
    dt, A = to_dev(dec["dt"]), to_dev(dec["A"])
    D = to_dev(dec["D"]) if with_D else None
    state = to_dev(dec["state"].astype(np.float16))
    T = dec["x16"].shape[0]
    ys = torch.empty((T,) + tuple(qx.shape[1:]), dtype=torch.float16, device=dev())
    for t in range(T):
        ssdq.state_update(state, qx[t], sx, qB[t], sB, qC[t], sC, dt[t], A, D, y=ys[t])
    torch.cuda.synchronize()
    return ys.float().cpu().numpy(), state.cpu().numpy().astype(np.float64)


def _small(seed, b, H, P, N, G, T):
    shape = workloads.DecodeShape(f"dec16_{seed}", b, T, H, P, N, G, 0.5)
    return _as_cache(workloads.make_decode(shape, seed_index=seed))


def _check(dec, y, st, tag=""):
    """Every step's y and the final cache of every (b, h) sequence against the oracle with the
    same caching, and the cache against the fp32-state recurrence; the oracle runs the sequences
    on host threads, each reduced to its maxima at once (nothing full-size is kept)."""
    c = oracle.decode_as_prefill(dec)
    T = dec["x16"].shape[0]

    def one(bh):
        b, h = bh
        y16, h16, _ = oracle.ssd_one(c, b, h, state_f16=True)
        _, h32, traj = oracle.ssd_one(c, b, h, chunk=1)    # traj: the state entering every step
        return (float(np.max(np.abs(h16))), float(np.max(np.abs(y16))),
                max(float(np.max(np.abs(traj))), float(np.max(np.abs(h32)))),
                float(np.max(np.abs(st[b, h] - h16))), float(np.max(np.abs(y[:, b, h] - y16))),
                float(np.max(np.abs(st[b, h] - h32))))

    r = np.array(threaded(one, [(b, h) for b in range(c.batch) for h in range(c.H)]))
    hmax, ymax, peak = r[:, 0].max(), r[:, 1].max(), r[:, 2].max()
    e_cache, e_y, e_fp32 = r[:, 3].max(), r[:, 4].max(), r[:, 5].max()
    note(f"{tag} ({len(r)} sequences) vs cached oracle: h {e_cache / hmax:.2e} "
         f"(spacings {e_cache / hmax / SPACING:.2f}), y {e_y / ymax:.2e}; vs fp32 state: {e_fp32 / peak:.2e} "
         f"of the peak (bound {T * 2.0 ** -11:.2e})")
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(st))
    assert e_cache <= FLIPS * SPACING * hmax
    assert e_y <= Y_TOL * ymax
    assert e_fp32 <= T * 2.0 ** -11 * peak + FLIPS * SPACING * hmax


@pytest.mark.parametrize("N,G", [(128, 4), (64, 2)])
def test_small_decode_every_step(N, G):
    dec = _small(60 + N, b=4, H=8, P=64, N=N, G=G, T=16)
    y, st = _gpu_decode_f16(dec)
    _check(dec, y, st, tag=f"f16 state N={N}")


def test_headdim_below_64_and_no_D():
    dec = _small(63, b=3, H=4, P=48, N=128, G=2, T=8)
    dec["D"] = None
    y, st = _gpu_decode_f16(dec, with_D=False)
    _check(dec, y, st, tag="f16 state P=48 no D")


def test_full_decode_workload():
    """batch 256, 128 heads, 8 groups, 128 steps on the 512 MiB binary16 state: every (batch,
    head) sequence against the oracle with the same caching."""
    note("generating decode workload")
    dec = _as_cache(workloads.make_decode("mamba2-8b-decode"))
    note("gpu decode 128 steps, binary16 state")
    y, st = _gpu_decode_f16(dec)
    note("oracle decode, binary16 state: all sequences")
    _check(dec, y, st, tag="f16 state full")
