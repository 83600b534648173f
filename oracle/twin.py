"""NumPy statement of the selective scan, used only to cross-check the C oracle.

TEST INFRASTRUCTURE ONLY.  Tiny shapes only: it materialises the discretised
(B, L, D, N) operands the way the Mamba walk-through's section 3.3 explains the
method (every Abar_t = exp(delta_t A) and every Bbar_t u_t formed up front, then
the state is advanced one timestep at a time), which is exactly what a fused
kernel must avoid at real sizes.
"""
from __future__ import annotations

from typing import Optional, Tuple

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
    section 3.1.4.2).  zoh: Bbar = (delta A)^-1 (exp(delta A) - 1) delta B
    (walk-through, section 2.2), here through scipy's exprel, (e^x - 1)/x."""
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
    a_bar = np.exp(da)
    b_bar = dl[:, :, :, None] * bm[:, :, None, :]
    if zoh:
        b_bar = scipy.special.exprel(da) * b_bar
    bu = b_bar * x[:, :, :, None]
    state = np.zeros((nb, nd, nn)) if h0 is None else np.array(h0, dtype=np.float64).reshape(nb, nd, nn)
    y = np.empty((nb, nl, nd))
    for t in range(nl):
        state = a_bar[:, t] * state + bu[:, t]
        y[:, t] = np.einsum("bdn,bn->bd", state, cm[:, t])
    if D is not None:
        y = y + np.asarray(D, dtype=np.float64)[None, None, :] * x
    if z is not None:
        zz = _f64(z)
        y = y * (zz / (1.0 + np.exp(-zz)))
    return y, state
