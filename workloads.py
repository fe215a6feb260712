"""Seeded synthetic workloads for the INT8-input Mamba-2 SSD scan.

This module only draws random inputs and derives the static calibration
scales from a separate calibration draw.  It holds none of the scan's
arithmetic (no quantizer, no recurrence), so that both the HIP path and the
CPU oracle can consume the same inputs without sharing any computation.

Shapes follow the Mamba-2 SSD layout (batch, length, heads, headdim) in which
the SSDi8 page shows the head axis carrying distinct activation patterns
(SSDi8, Figure 2).  The scale granularity is the one the pages use: one static
scale per head for x and one per state group for B and C (Quamba2 rebuttal,
"per-state-group quantization"; SSDi8, Table 10 "per-H(G)"), calibrated once
offline as absmax/127 over a separate calibration draw (Quamba project page,
"static per-tensor quantization" generalised per head / per group).

The pages measure on real Mamba-2 activations (LAMBADA, Wikitext2, Pile, ...);
none of those datasets or checkpoints is available, so these seeded draws stand
in for them with the model shapes the pages name (Mamba-2 1.3B: d_inner 4096 =
64 heads x 64; 2.7B: 80 heads, one B/C group; 8B: 128 heads, 8 groups).

Random-number recipe (seeds per workload k): model seed 100+k, data seed 200+k,
calibration seed 300+k; numpy PCG64.  Large arrays are drawn directly in
float32 (numpy's float32 normal sampler) and then cast to float16.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class PrefillShape:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    x_dist: str          # "normal" | "outlier_heads" | "lognormal_heads"
    dt_dist: str         # "fixed_bias" (softplus(N(-2,0.5))) | "head_bias" (softplus(N(0,0.5)+b_h))
    h0_std: float = 0.0  # 0 -> no initial state

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


@dataclasses.dataclass(frozen=True)
class DecodeShape:
    name: str
    batch: int
    steps: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    state_std: float
    x_dist: str = "lognormal_heads"
    dt_dist: str = "head_bias"


# The five workloads: a tiny one, three prefill shapes, one decode shape.
WORKLOADS = {
    "tiny": PrefillShape("tiny", 1, 256, 4, 16, 16, 1, 64, "normal", "fixed_bias"),
    "mamba2-1.3b-prefill": PrefillShape("mamba2-1.3b-prefill", 4, 2048, 64, 64, 128, 1, 256,
                                        "outlier_heads", "fixed_bias"),
    "mamba2-2.7b-long-prefill": PrefillShape("mamba2-2.7b-long-prefill", 1, 16384, 80, 64, 128, 1, 256,
                                             "outlier_heads", "fixed_bias", h0_std=0.1),
    "mamba2-8b-prefill": PrefillShape("mamba2-8b-prefill", 8, 4096, 128, 64, 128, 8, 256,
                                      "lognormal_heads", "head_bias"),
    "mamba2-8b-decode": DecodeShape("mamba2-8b-decode", 256, 128, 128, 64, 128, 8, 0.5),
}
WORKLOAD_ORDER = ["tiny", "mamba2-1.3b-prefill", "mamba2-2.7b-long-prefill",
                  "mamba2-8b-prefill", "mamba2-8b-decode"]
SEED_INDEX = {name: k for k, name in enumerate(WORKLOAD_ORDER)}


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _softplus(z: np.ndarray) -> np.ndarray:
    # numerically safe log(1 + exp(z)); dt is handed to the scan already softplus'd
    return np.logaddexp(0.0, z)


@dataclasses.dataclass
class ModelParams:
    A: np.ndarray          # [H] float32, <= 0
    D: np.ndarray          # [H] float32
    x_mag: np.ndarray      # [H] float64 per-head magnitude of x
    dt_bias: np.ndarray    # [H] float64 (zeros for the fixed-bias recipe)


def model_params(nheads: int, x_dist: str, dt_dist: str, seed: int) -> ModelParams:
    """Per-head properties shared by the calibration and the test draw."""
    rng = _rng(seed)
    A = (-np.exp(rng.uniform(0.0, math.log(16.0), size=nheads))).astype(np.float32)
    D = rng.uniform(0.5, 1.5, size=nheads).astype(np.float32)
    x_mag = np.ones(nheads)
    if x_dist == "outlier_heads":
        n_out = int(round(0.1 * nheads))
        heads = rng.choice(nheads, size=n_out, replace=False)
        x_mag[heads] = 20.0
    elif x_dist == "lognormal_heads":
        x_mag = np.exp(rng.normal(0.0, 1.0, size=nheads))
    elif x_dist != "normal":
        raise ValueError(x_dist)
    dt_bias = np.zeros(nheads)
    if dt_dist == "head_bias":
        dt_bias = rng.uniform(-4.0, -1.0, size=nheads)
    elif dt_dist != "fixed_bias":
        raise ValueError(dt_dist)
    return ModelParams(A, D, x_mag, dt_bias)


def _draw_activations(rng, lead: tuple, nheads, headdim, ngroups, dstate, params: ModelParams):
    x = rng.standard_normal(size=lead + (nheads, headdim), dtype=np.float32)
    x *= params.x_mag.astype(np.float32)[:, None]
    B = rng.standard_normal(size=lead + (ngroups, dstate), dtype=np.float32)
    C = rng.standard_normal(size=lead + (ngroups, dstate), dtype=np.float32)
    return x.astype(np.float16), B.astype(np.float16), C.astype(np.float16)


def _draw_dt(rng, lead: tuple, nheads, params: ModelParams, dt_dist: str) -> np.ndarray:
    if dt_dist == "fixed_bias":
        z = rng.normal(-2.0, 0.5, size=lead + (nheads,))
    else:
        z = rng.normal(0.0, 0.5, size=lead + (nheads,)) + params.dt_bias
    return _softplus(z).astype(np.float32)


def absmax_scale(t16: np.ndarray, axis_keep: int) -> np.ndarray:
    """Static scale per index of `axis_keep` (heads for x, groups for B/C):
    fp32(absmax over the calibration tensor) / 127, or 1 where the absmax is 0."""
    t = np.abs(t16.astype(np.float32))
    axes = tuple(i for i in range(t.ndim) if i != (axis_keep % t.ndim))
    amax = t.max(axis=axes).astype(np.float32)
    s = amax / np.float32(127.0)
    s[amax == 0] = np.float32(1.0)
    return s.astype(np.float32)


def absmax_scale_per_state(t16: np.ndarray) -> np.ndarray:
    """Static scale per (group, state) of a B or C calibration tensor (..., G, N): fp32(absmax over
    the leading axes) / 127, or 1 where it is 0 (SSDi8 Table 10: per-P(N) together with per-H(G))."""
    t = np.abs(t16.astype(np.float32))
    amax = t.reshape(-1, t.shape[-2], t.shape[-1]).max(axis=0).astype(np.float32)
    s = amax / np.float32(127.0)
    s[amax == 0] = np.float32(1.0)
    return s.astype(np.float32)


def percentile_scale(t16: np.ndarray, axis_keep: int, q: float) -> np.ndarray:
    """Static scale per index of `axis_keep` with percentile clipping (the calibration of x the
    Quamba2 rebuttal compares in Table R9): fp32(the q-th percentile of |t| over the calibration
    tensor for that index) / 127, or 1 where it is 0.  Values beyond it saturate to +-127."""
    t = np.abs(t16.astype(np.float32))
    keep = axis_keep % t.ndim
    moved = np.moveaxis(t, keep, 0).reshape(t.shape[keep], -1)
    amax = np.percentile(moved, q, axis=1).astype(np.float32)
    s = amax / np.float32(127.0)
    s[amax == 0] = np.float32(1.0)
    return s.astype(np.float32)


def cluster_channel_scales(x16: np.ndarray, nclusters: int) -> np.ndarray:
    """Static x scales per (head, channel) from channel clusters of an x calibration tensor
    (..., H, P) -- the reading taken of Quamba2's sort-and-cluster, whose pages name the step but
    give no algorithm: per head, the channels sorted by their calibration absmax are cut into
    `nclusters` runs of consecutive sorted order (sizes as equal as possible, the largest channels
    last), and every channel of a run takes the run's absmax / 127 (1 where it is 0).  Returns
    (H, P) fp32; nclusters = 1 gives the per-head absmax scale on every channel, nclusters = P
    one absmax scale per channel."""
    t = np.abs(x16.astype(np.float32))
    H, P = t.shape[-2], t.shape[-1]
    if not 1 <= nclusters <= P:
        raise ValueError("nclusters must be in 1..headdim")
    amax = t.reshape(-1, H, P).max(axis=0)                     # (H, P)
    out = np.empty((H, P), np.float32)
    bounds = [(k * P) // nclusters for k in range(nclusters + 1)]
    for h in range(H):
        order = np.argsort(amax[h], kind="stable")
        for k in range(nclusters):
            members = order[bounds[k]:bounds[k + 1]]
            m = np.float32(amax[h, members].max())
            out[h, members] = m / np.float32(127.0) if m > 0 else np.float32(1.0)
    return out


def make_prefill(shape: PrefillShape | str, seed_index: int | None = None, batch: int | None = None,
                 seqlen: int | None = None) -> dict:
    """Seeded prefill inputs.  `batch`/`seqlen` may shrink the test draw (the
    calibration draw keeps the workload's shape unless it is larger than the
    test draw would be, in which case it is shrunk the same way)."""
    if isinstance(shape, str):
        shape = WORKLOADS[shape]
    k = SEED_INDEX.get(shape.name, 0) if seed_index is None else seed_index
    b = shape.batch if batch is None else batch
    L = shape.seqlen if seqlen is None else seqlen
    H, P, N, G = shape.nheads, shape.headdim, shape.dstate, shape.ngroups
    params = model_params(H, shape.x_dist, shape.dt_dist, 100 + k)

    cal = _rng(300 + k)
    xc, Bc, Cc = _draw_activations(cal, (b, L), H, P, G, N, params)
    sx, sB, sC = absmax_scale(xc, -2), absmax_scale(Bc, -2), absmax_scale(Cc, -2)
    del xc, Bc, Cc

    rng = _rng(200 + k)
    x, B, C = _draw_activations(rng, (b, L), H, P, G, N, params)
    dt = _draw_dt(rng, (b, L), H, params, shape.dt_dist)
    h0 = None
    if shape.h0_std > 0:
        h0 = (rng.standard_normal(size=(b, H, P, N), dtype=np.float32) * np.float32(shape.h0_std))
    return dict(x16=x, B16=B, C16=C, dt=dt, A=params.A, D=params.D, h0=h0,
                x_scale=sx, B_scale=sB, C_scale=sC,
                batch=b, seqlen=L, nheads=H, headdim=P, dstate=N, ngroups=G, chunk=shape.chunk)


def make_calibrated_pair(shape: PrefillShape, seed_index: int, x_mean: float = 0.0,
                         x_clip_pct: float | None = None, bc_per_state: bool = False,
                         state_spread: float = 0.0, channel_spread: float = 0.0,
                         x_clusters: int | None = None) -> tuple[dict, dict]:
    """A calibration draw and a test draw of one prefill shape that share the model's per-head
    properties and the static scales calibrated on the first: (cal, test), each in make_prefill's
    format.  x = m_h (N(0, 1) + x_mean), so a nonzero x_mean makes the activations one-sided; with
    x_clip_pct the x scales clip at that percentile of |x| (percentile_scale), else absmax / 127,
    so the test draw's x codes saturate where it exceeds the calibrated range.  With bc_per_state
    the B and C scales are one per (group, state) (absmax_scale_per_state); state_spread > 0 gives
    every state column of B and C its own magnitude exp(N(0, state_spread)) (drawn by the model
    seed), the case those scales are for.  channel_spread > 0 likewise gives every x channel of
    every head its own magnitude exp(N(0, channel_spread)), and x_clusters = k calibrates x with
    one scale per (head, channel cluster) (cluster_channel_scales: an (H, P) table).  The
    calibration draw also carries dt (and h0, when the shape has one), so that a scan can be run
    over it."""
    k = seed_index
    b, L, H, P, N, G = shape.batch, shape.seqlen, shape.nheads, shape.headdim, shape.dstate, shape.ngroups
    params = model_params(H, shape.x_dist, shape.dt_dist, 100 + k)
    col = np.ones((2, G, N), np.float32)
    if state_spread > 0:
        col = np.exp(_rng(500 + k).normal(0.0, state_spread, size=(2, G, N))).astype(np.float32)
    chan = None
    if channel_spread > 0:
        chan = np.exp(_rng(600 + k).normal(0.0, channel_spread, size=(H, P))).astype(np.float32)

    def draw(seed):
        rng = _rng(seed)
        x, B, C = _draw_activations(rng, (b, L), H, P, G, N, params)
        if state_spread > 0:
            B = (B.astype(np.float32) * col[0]).astype(np.float16)
            C = (C.astype(np.float32) * col[1]).astype(np.float16)
        if chan is not None:
            x = (x.astype(np.float32) * chan).astype(np.float16)
        if x_mean:
            x = (x.astype(np.float32) + np.float32(x_mean) * params.x_mag.astype(np.float32)[:, None]).astype(np.float16)
        dt = _draw_dt(rng, (b, L), H, params, shape.dt_dist)
        h0 = None
        if shape.h0_std > 0:
            h0 = rng.standard_normal(size=(b, H, P, N), dtype=np.float32) * np.float32(shape.h0_std)
        return dict(x16=x, B16=B, C16=C, dt=dt, A=params.A, D=params.D, h0=h0,
                    batch=b, seqlen=L, nheads=H, headdim=P, dstate=N, ngroups=G, chunk=shape.chunk)

    cal, test = draw(300 + k), draw(200 + k)
    if x_clusters is not None:
        sx = cluster_channel_scales(cal["x16"], x_clusters)
    else:
        sx = absmax_scale(cal["x16"], -2) if x_clip_pct is None else percentile_scale(cal["x16"], -2, x_clip_pct)
    bc = absmax_scale_per_state if bc_per_state else (lambda t: absmax_scale(t, -2))
    scales = dict(x_scale=sx, B_scale=bc(cal["B16"]), C_scale=bc(cal["C16"]))
    cal.update(scales)
    test.update(scales)
    return cal, test


def make_frontend(shape: PrefillShape | str, seed_index: int | None = None, batch: int | None = None,
                  seqlen: int | None = None) -> dict:
    """Seeded inputs of the block's front end for a prefill shape: the in-projection output xBC
    (b, L, H*P + 2*G*N) fp16 with channels [x | B | C] (the prefill draw's activations), depthwise
    conv taps (C, 4) close to a pass-through of the newest token (tap 3 ~ 1 + N(0, 0.05), the
    older taps ~ N(0, 0.1)) and a small bias, all fp16-representable fp32, raw dt ~ N(-4, 1) with
    a per-head dt_bias ~ U(-0.5, 0.5), and the prefill draw's static x/B/C scales."""
    inp = make_prefill(shape, seed_index, batch, seqlen)
    b, L = inp["batch"], inp["seqlen"]
    H, P, N, G = inp["nheads"], inp["headdim"], inp["dstate"], inp["ngroups"]
    xbc = np.concatenate([inp["x16"].reshape(b, L, H * P), inp["B16"].reshape(b, L, G * N),
                          inp["C16"].reshape(b, L, G * N)], axis=2)
    C = xbc.shape[2]
    name = shape if isinstance(shape, str) else shape.name
    k = SEED_INDEX.get(name, 0) if seed_index is None else seed_index
    rng = _rng(400 + k)
    w = rng.standard_normal((C, 4)).astype(np.float32) * np.float32(0.1)
    w[:, 3] = 1.0 + rng.standard_normal(C).astype(np.float32) * np.float32(0.05)
    w = w.astype(np.float16).astype(np.float32)
    bias = (rng.standard_normal(C) * 0.02).astype(np.float16).astype(np.float32)
    dt_raw = (rng.standard_normal((b, L, H)) - 4.0).astype(np.float32)
    dt_bias = rng.uniform(-0.5, 0.5, H).astype(np.float32)
    return dict(xbc16=np.ascontiguousarray(xbc), conv_w=w, conv_b=bias, dt_raw=dt_raw, dt_bias=dt_bias,
                x_scale=inp["x_scale"], B_scale=inp["B_scale"], C_scale=inp["C_scale"], A=inp["A"], D=inp["D"],
                batch=b, seqlen=L, nheads=H, headdim=P, dstate=N, ngroups=G, chunk=inp["chunk"])


def make_decode(shape: DecodeShape | str, seed_index: int | None = None, batch: int | None = None,
                steps: int | None = None) -> dict:
    """Seeded decode inputs: an fp32 state (b,H,P,N) and `steps` tokens per sequence.
    Per-step activations are stacked on a leading step axis: x16 (steps,b,H,P),
    B16/C16 (steps,b,G,N), dt (steps,b,H)."""
    if isinstance(shape, str):
        shape = WORKLOADS[shape]
    k = SEED_INDEX.get(shape.name, 4) if seed_index is None else seed_index
    b = shape.batch if batch is None else batch
    T = shape.steps if steps is None else steps
    H, P, N, G = shape.nheads, shape.headdim, shape.dstate, shape.ngroups
    params = model_params(H, shape.x_dist, shape.dt_dist, 100 + k)

    cal = _rng(300 + k)
    xc, Bc, Cc = _draw_activations(cal, (T, b), H, P, G, N, params)
    sx, sB, sC = absmax_scale(xc, -2), absmax_scale(Bc, -2), absmax_scale(Cc, -2)
    del xc, Bc, Cc

    rng = _rng(200 + k)
    state = rng.standard_normal(size=(b, H, P, N), dtype=np.float32) * np.float32(shape.state_std)
    x, B, C = _draw_activations(rng, (T, b), H, P, G, N, params)
    dt = _draw_dt(rng, (T, b), H, params, shape.dt_dist)
    return dict(state=state, x16=x, B16=B, C16=C, dt=dt, A=params.A, D=params.D,
                x_scale=sx, B_scale=sB, C_scale=sC,
                batch=b, steps=T, nheads=H, headdim=P, dstate=N, ngroups=G)


def make_custom_prefill(seed: int, batch: int, seqlen: int, nheads: int, headdim: int, dstate: int,
                        ngroups: int, chunk: int, x_dist: str = "normal", dt_dist: str = "fixed_bias",
                        h0_std: float = 0.0) -> dict:
    """A prefill draw of any shape (used for ragged and edge-case tests)."""
    shape = PrefillShape(f"custom{seed}", batch, seqlen, nheads, headdim, dstate, ngroups, chunk,
                         x_dist, dt_dist, h0_std)
    return make_prefill(shape, seed_index=seed)
