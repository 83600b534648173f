"""NumPy statement of the selective scan, used only to cross-check the C oracle.

TEST INFRASTRUCTURE ONLY.  Tiny shapes only: it forms the discretised operands
Abar_t = exp(delta_t A) and Bbar_t u_t for every (b, t, d, n), then solves the
recurrence h_t = Abar_t h_{t-1} + Bbar_t u_t not step by step but as an inclusive
scan of the affine maps h -> a h + c by recursive doubling (the parallel scan over
an associative operator of the LTI chapter, section 3.1.5.2): after the round with
offset k, entry t holds the composition of the maps of steps max(0, t-2k+1) .. t,
combined earlier map first, (a1, c1) then (a2, c2) -> (a2 a1, a2 c1 + c2).  After
ceil(log2 L) rounds entry t maps h0 to h_t.  The C oracle's sequential loop shares
neither the order of operations nor any code with this.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np
import scipy.special


def _f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def twin_scan(u, delta, A, B, C, D=None, z=None, h0=None, *, delta_bias=None, delta_softplus=False,
              zoh=False) -> Tuple[np.ndarray, np.ndarray]:
    """Return (y (B,L,D), h_last (B,D,N)) in float64.

    delta_bias / delta_softplus: step size softplus(delta + bias[d]) (LTI chapter,
    section 3.1.4.2), here numpy's logaddexp(0, v).  zoh: Bbar = (delta A)^-1 (exp(delta
    A) - 1) delta B (walk-through, section 2.2), here through scipy's exprel, (e^x - 1)/x."""
    x = _f64(u)
    dl = _f64(delta)
    if delta_bias is not None:
        dl = dl + np.asarray(delta_bias, dtype=np.float64)[None, None, :]
    if delta_softplus:
        dl = np.logaddexp(0.0, dl)  # log(e^0 + e^v) = log(1 + e^v)
    a = _f64(A)
    bm = _f64(B)
    cm = _f64(C)
    nb, nl, nd = x.shape
    nn = a.shape[1]
    # discretised operands for all (b, t, d, n)
    da = dl[:, :, :, None] * a[None, None, :, :]
    abar = np.exp(da)
    bbar = dl[:, :, :, None] * bm[:, :, None, :]
    if zoh:
        bbar = scipy.special.exprel(da) * bbar
    # the map of step t: h -> abar_t h + c_t
    P = abar
    S = bbar * x[:, :, :, None]
    k = 1
    while k < nl:
        # compose every entry t >= k with entry t - k (the earlier map first)
        P_new = P.copy()
        S_new = S.copy()
        P_new[:, k:] = P[:, k:] * P[:, :-k]
        S_new[:, k:] = P[:, k:] * S[:, :-k] + S[:, k:]
        P, S = P_new, S_new
        k *= 2
    start = np.zeros((nb, nd, nn)) if h0 is None else np.array(h0, dtype=np.float64).reshape(nb, nd, nn)
    h = P * start[:, None, :, :] + S  # (B, L, D, N): the state after every step
    y = np.sum(h * cm[:, :, None, :], axis=3)
    if D is not None:
        y = y + np.asarray(D, dtype=np.float64)[None, None, :] * x
    if z is not None:
        zz = _f64(z)
        y = y * (zz / (1.0 + np.exp(-zz)))
    return y, h[:, -1]
