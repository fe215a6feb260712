"""Independent chunked (state-space-duality) evaluation in numpy float64.

Test-only second implementation used to pin the sequential oracle.  It does not
step token by token: within each chunk it forms the masked "attention" matrix
(the dual form the SSDi8 abstract refers to as the attention mode of SSD),

    y_diag = (L o (C B^T)) (dt o x),   L[l, j] = exp(Acs_l - Acs_j) for j <= l, else 0,

carries the inter-chunk state with one matrix update per chunk,

    H_{c+1} = exp(Acs_last) H_c + sum_j exp(Acs_last - Acs_j) dt_j x_j B_j^T,

and reads the carried state out with y_off[l] = exp(Acs_l) C_l . H_c.  With
chunk = L this is the textbook quadratic dual of the whole sequence; with
chunk = 1 it is the recurrence again.  Vectorised over all (batch, head) pairs.
"""
from __future__ import annotations

import numpy as np


def dequantize(qx, sx, qB, sB, qC, sC):
    """Dequantized float64 inputs, with B and C broadcast from groups to heads."""
    x = qx.astype(np.float64) * sx.astype(np.float64)[:, None]           # (b, L, H, P)
    B = qB.astype(np.float64) * sB.astype(np.float64)[:, None]           # (b, L, G, N)
    C = qC.astype(np.float64) * sC.astype(np.float64)[:, None]
    H, G = qx.shape[2], qB.shape[2]
    rep = H // G
    B = np.repeat(B, rep, axis=2)                                         # (b, L, H, N)
    C = np.repeat(C, rep, axis=2)
    return x, B, C


def chunked_ssd(qx, sx, qB, sB, qC, sC, dt, A, D=None, h0=None, chunk=64):
    """Returns dict(y (b,L,H,P), h_final (b,H,P,N), Acs (b,H,nc,Q) NaN-padded,
    S (b,nc,H,P,N) chunk states, Hprev (b,nc,H,P,N) states entering each chunk)."""
    x, B, C = dequantize(qx, sx, qB, sB, qC, sC)
    b, L, H, P = x.shape
    N = B.shape[-1]
    dt = dt.astype(np.float64)
    A = A.astype(np.float64)
    nc = -(-L // chunk)
    Hs = np.zeros((b, H, P, N)) if h0 is None else h0.astype(np.float64).copy()
    y = np.empty((b, L, H, P))
    Acs_out = np.full((b, H, nc, chunk), np.nan)
    S_out = np.empty((b, nc, H, P, N))
    Hprev_out = np.empty((b, nc, H, P, N))
    for c in range(nc):
        lo, hi = c * chunk, min(L, (c + 1) * chunk)
        q = hi - lo
        dA = dt[:, lo:hi, :] * A[None, None, :]                          # (b, q, H)
        Acs = np.cumsum(dA, axis=1)                                       # (b, q, H)
        Acs_out[:, :, c, :q] = np.transpose(Acs, (0, 2, 1))
        # decay mask L[b, H, l, j]
        diff = Acs.transpose(0, 2, 1)[:, :, :, None] - Acs.transpose(0, 2, 1)[:, :, None, :]
        causal = np.tril(np.ones((q, q), dtype=bool))
        Lmask = np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0)
        xc, Bc, Cc = x[:, lo:hi], B[:, lo:hi], C[:, lo:hi]
        dtc = dt[:, lo:hi]
        CB = np.einsum("blhn,bjhn->bhlj", Cc, Bc)
        xdt = xc * dtc[..., None]                                         # (b, q, H, P)
        y_diag = np.einsum("bhlj,bjhp->blhp", CB * Lmask, xdt)
        y_off = np.einsum("blhn,bhpn->blhp", Cc, Hs) * np.exp(Acs)[..., None]
        y[:, lo:hi] = y_diag + y_off
        Hprev_out[:, c] = Hs
        w = np.exp(Acs[:, -1:, :] - Acs) * dtc                             # (b, q, H): LUT_state
        S = np.einsum("bjh,bjhp,bjhn->bhpn", w, xc, Bc)
        S_out[:, c] = S
        Hs = np.exp(Acs[:, -1, :])[:, :, None, None] * Hs + S
    if D is not None:
        y = y + D.astype(np.float64)[None, None, :, None] * x
    return dict(y=y, h_final=Hs, Acs=Acs_out, S=S_out, Hprev=Hprev_out)
