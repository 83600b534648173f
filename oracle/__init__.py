"""CPU oracle for the selective scan -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the bench's CPU-baseline leg may
import this package.  The library path never does.

* ``scan`` / ``step`` call the plain fp64 C loop in ``ss_oracle.c``
  (Mamba walk-through section 3.3 ``selective_scan`` plus the block's D skip and
  silu(z) gate, section 3.4).  Options: ``delta_bias`` / ``delta_softplus``
  (step size softplus(delta + bias[d]), LTI chapter section 3.1.4.2) and ``zoh``
  (zero-order-hold Bbar of the walk-through's section 2.2).
* ``scan_bwd`` calls the fp64 backward in ``ss_oracle.c``: the chain rule taken
  backward through the same recurrence, every state recomputed per lane.
* ``conv1d_silu`` calls the fp64 causal depthwise convolution + SiLU of the Mamba
  block (walk-through section 3.4) that produces the scan's u.
* ``ssd`` calls the fp64 multi-head recurrence of Mamba-2 (walk-through sections 4.1
  and 5.2): an (N, P) state per head, scalar decay exp(dt A) per head.
* ``twin_scan`` (in ``twin.py``) is an independent NumPy statement of the same
  definition, used only to cross-check the C loop on tiny shapes.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, the LTI convolution identity, brute force, invariants and a
hand-worked fixture); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ss_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
SOFTPLUS, ZOH = 1, 2  # option flags of oracle_scan / oracle_step
_lib = None


def build(force: bool = True) -> str:
    """Compile ss_oracle.c into liboracle.so next to it (gcc, -O2, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared",
               "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class OracleLib:
    """ctypes view of one compiled oracle library (the default one, or a test build)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        vp, i64, ip = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.oracle_scan.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ip, ip, i64, i64, i64, i64,
                                    vp, i64, vp, vp, vp, i64, vp, ip]
        lib.oracle_scan.restype = ctypes.c_int
        lib.oracle_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ip, ip, i64, i64, i64, vp, i64, vp, ip]
        lib.oracle_step.restype = ctypes.c_int
        lib.oracle_scan_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ip, ip, i64, i64, i64, i64,
                                        vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ip]
        lib.oracle_scan_bwd.restype = ctypes.c_int
        lib.oracle_conv1d_silu.argtypes = [vp, i64, vp, vp, ip, i64, i64, i64, i64, vp]
        lib.oracle_conv1d_silu.restype = ctypes.c_int
        lib.oracle_ssd.argtypes = [vp, vp, vp, vp, vp, vp, vp, ip, i64, i64, i64, i64, i64, vp, i64, vp, vp, ip]
        lib.oracle_ssd.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def scan(self, *args, **kwargs):
        return scan(*args, _lib=self.lib, **kwargs)

    def step(self, *args, **kwargs):
        return step(*args, _lib=self.lib, **kwargs)

    def scan_bwd(self, *args, **kwargs):
        return scan_bwd(*args, _lib=self.lib, **kwargs)

    def conv1d_silu(self, *args, **kwargs):
        return conv1d_silu(*args, _lib=self.lib, **kwargs)

    def ssd(self, *args, **kwargs):
        return ssd(*args, _lib=self.lib, **kwargs)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = OracleLib(_LIB).lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_of(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("operand dtype must be float32 or uint16 (bf16 bits), got %s" % a.dtype)


def _c(a: Optional[np.ndarray], dt=None) -> Optional[np.ndarray]:
    if a is None:
        return None
    return np.ascontiguousarray(a if dt is None else a.astype(dt, copy=False))


def _flags(delta_softplus: bool, zoh: bool) -> int:
    return (SOFTPLUS if delta_softplus else 0) | (ZOH if zoh else 0)


def scan(u: np.ndarray, delta: np.ndarray, A: np.ndarray, B: np.ndarray, C: np.ndarray,
         D: Optional[np.ndarray] = None, z: Optional[np.ndarray] = None,
         h0: Optional[np.ndarray] = None, lanes: Optional[Sequence[int]] = None,
         record_t: Optional[Sequence[int]] = None, threads: int = 1, *,
         delta_bias: Optional[np.ndarray] = None, delta_softplus: bool = False, zoh: bool = False,
         _lib=None) -> Dict[str, np.ndarray]:
    """fp64 scan.  u, delta, z: (B,L,D); B, C: (B,L,N) in float32 or bf16 bits (uint16);
    A (D,N), D (D,) and delta_bias (D,) float32; h0 (B,D,N) any float (widened to double).

    Returns ``y`` (B,L,D) -- or (n_lanes, L) when ``lanes`` (flat b*D+d) is given --
    ``h_last`` (B,D,N) / (n_lanes, N), and ``h_rec`` (n_lanes, len(record_t), N) with the
    state right after each timestep in ``record_t``.
    """
    lib = _lib or _load()
    dt = _dtype_of(u)
    batch, seqlen, dim = u.shape
    dstate = A.shape[1]
    for name, arr, shp in (("delta", delta, u.shape), ("B", B, (batch, seqlen, dstate)),
                           ("C", C, (batch, seqlen, dstate))):
        if tuple(arr.shape) != tuple(shp) or _dtype_of(arr) != dt:
            raise ValueError("%s has shape %s dtype %s" % (name, arr.shape, arr.dtype))
    if z is not None and (tuple(z.shape) != tuple(u.shape) or _dtype_of(z) != dt):
        raise ValueError("z mismatch")
    u, delta, B, C, z = _c(u), _c(delta), _c(B), _c(C), _c(z)
    A = _c(A, np.float32)
    D = _c(D, np.float32)
    bias = _c(delta_bias, np.float32)
    h0 = _c(h0, np.float64)
    lane_arr = None if lanes is None else np.ascontiguousarray(np.asarray(lanes, dtype=np.int64))
    n_lanes = batch * dim if lane_arr is None else lane_arr.size
    rec = None if record_t is None else np.ascontiguousarray(np.asarray(record_t, dtype=np.int64))
    n_rec = 0 if rec is None else rec.size
    y = np.empty((n_lanes, seqlen), dtype=np.float64)
    h_last = np.empty((n_lanes, dstate), dtype=np.float64)
    h_rec = np.empty((n_lanes, max(n_rec, 1), dstate), dtype=np.float64)
    rc = lib.oracle_scan(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                         _ptr(bias), _flags(delta_softplus, zoh), dt, batch, seqlen, dim, dstate, _ptr(lane_arr), n_lanes,
                         _ptr(y), _ptr(h_last), _ptr(rec), n_rec,
                         _ptr(h_rec) if rec is not None else None, int(threads))
    if rc != 0:
        raise ValueError("oracle_scan rejected its arguments")
    out = {"h_rec": h_rec[:, :n_rec]}
    if lane_arr is None:
        out["y"] = y.reshape(batch, dim, seqlen).transpose(0, 2, 1).copy()
        out["h_last"] = h_last.reshape(batch, dim, dstate)
    else:
        out["y"] = y
        out["h_last"] = h_last
    return out


def step(h: np.ndarray, u: np.ndarray, delta: np.ndarray, A: np.ndarray, B: np.ndarray,
         C: np.ndarray, D: Optional[np.ndarray] = None, z: Optional[np.ndarray] = None,
         lanes: Optional[Sequence[int]] = None, *, delta_bias: Optional[np.ndarray] = None,
         delta_softplus: bool = False, zoh: bool = False, threads: int = 1, _lib=None) -> np.ndarray:
    """One recurrent token.  h: float64 (B,D,N), or (n_lanes, N) with ``lanes``; updated
    in place.  u, delta, z: (B,D); B, C: (B,N).  Returns y float64 (B,D) / (n_lanes,).
    ``threads`` > 1 splits the lanes over threads (bit-identical results)."""
    lib = _lib or _load()
    if h.dtype != np.float64 or not h.flags.c_contiguous:
        raise TypeError("h must be a C-contiguous float64 array (updated in place)")
    dt = _dtype_of(u)
    batch, dim = u.shape
    dstate = A.shape[1]
    u, delta, B, C, z = _c(u), _c(delta), _c(B), _c(C), _c(z)
    A = _c(A, np.float32)
    D = _c(D, np.float32)
    bias = _c(delta_bias, np.float32)
    lane_arr = None if lanes is None else np.ascontiguousarray(np.asarray(lanes, dtype=np.int64))
    n_lanes = batch * dim if lane_arr is None else lane_arr.size
    if h.size != n_lanes * dstate:
        raise ValueError("h has %d values, expected %d" % (h.size, n_lanes * dstate))
    y = np.empty(n_lanes, dtype=np.float64)
    rc = lib.oracle_step(_ptr(h), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                         _ptr(bias), _flags(delta_softplus, zoh), dt, batch, dim, dstate, _ptr(lane_arr), n_lanes, _ptr(y),
                         int(threads))
    if rc != 0:
        raise ValueError("oracle_step rejected its arguments")
    return y.reshape(batch, dim) if lane_arr is None else y


def scan_bwd(u: np.ndarray, delta: np.ndarray, A: np.ndarray, B: np.ndarray, C: np.ndarray,
             D: Optional[np.ndarray] = None, z: Optional[np.ndarray] = None,
             h0: Optional[np.ndarray] = None, *, dy: np.ndarray, dh_last: Optional[np.ndarray] = None,
             delta_bias: Optional[np.ndarray] = None, delta_softplus: bool = False, zoh: bool = False,
             threads: int = 1, _lib=None) -> Dict[str, np.ndarray]:
    """fp64 gradients of sum(dy * y) + sum(dh_last * h_last) with respect to every input of
    ``scan`` (same argument conventions and options; dy (B,L,D) and dh_last (B,D,N) any float).

    Returns float64 ``du``, ``ddelta``, ``dz`` (B,L,D); ``dA`` (D,N); ``dB``, ``dC`` (B,L,N);
    ``dD``, ``ddelta_bias`` (D,); ``dh0`` (B,D,N).  Gradients of absent inputs are absent
    (``dz`` without z, ``dD`` without D, ``ddelta_bias`` without a bias).  ``ddelta`` is with
    respect to delta as passed (the raw value under ``delta_softplus``).
    """
    lib = _lib or _load()
    dt = _dtype_of(u)
    batch, seqlen, dim = u.shape
    dstate = A.shape[1]
    for name, arr, shp in (("delta", delta, u.shape), ("B", B, (batch, seqlen, dstate)),
                           ("C", C, (batch, seqlen, dstate))):
        if tuple(arr.shape) != tuple(shp) or _dtype_of(arr) != dt:
            raise ValueError("%s has shape %s dtype %s" % (name, arr.shape, arr.dtype))
    u, delta, B, C, z = _c(u), _c(delta), _c(B), _c(C), _c(z)
    A = _c(A, np.float32)
    D = _c(D, np.float32)
    bias = _c(delta_bias, np.float32)
    h0 = _c(h0, np.float64)
    dy = _c(dy, np.float64)
    dhl = _c(dh_last, np.float64)
    if dy.shape != (batch, seqlen, dim):
        raise ValueError("dy must be (B, L, D)")
    out = {k: np.zeros((batch, seqlen, dim)) for k in ("du", "ddelta", "dz")}
    out["dA"] = np.zeros((dim, dstate))
    out["dB"] = np.zeros((batch, seqlen, dstate))
    out["dC"] = np.zeros((batch, seqlen, dstate))
    out["dD"] = np.zeros(dim)
    out["ddelta_bias"] = np.zeros(dim)
    out["dh0"] = np.zeros((batch, dim, dstate))
    rc = lib.oracle_scan_bwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                             _ptr(bias), _flags(delta_softplus, zoh), dt, batch, seqlen, dim, dstate,
                             _ptr(dy), _ptr(dhl), _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dz"]),
                             _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]),
                             _ptr(out["ddelta_bias"]), _ptr(out["dh0"]), int(threads))
    if rc != 0:
        raise ValueError("oracle_scan_bwd rejected its arguments")
    if z is None:
        del out["dz"]
    if D is None:
        del out["dD"]
    if bias is None:
        del out["ddelta_bias"]
    return out


def conv1d_silu(x: np.ndarray, weight: np.ndarray, bias: Optional[np.ndarray] = None, *, dim: Optional[int] = None,
                _lib=None) -> np.ndarray:
    """fp64 causal depthwise convolution + SiLU.  x: (B, L, S) float32 or bf16 bits with the
    channels in its first ``dim`` columns (default S: all of them; e.g. the x half of a
    (B, L, 2D) projection with dim = D); weight (dim, width), bias (dim,) float32.
    Returns u (B, L, dim) float64."""
    lib = _lib or _load()
    dt = _dtype_of(x)
    x = _c(x)
    batch, seqlen, stride = x.shape
    dim = stride if dim is None else int(dim)
    weight = _c(weight, np.float32)
    width = weight.shape[1]
    if weight.shape != (dim, width):
        raise ValueError("weight must be (dim, width)")
    bias = _c(bias, np.float32)
    u = np.empty((batch, seqlen, dim), dtype=np.float64)
    rc = lib.oracle_conv1d_silu(_ptr(x), stride, _ptr(weight), _ptr(bias), dt, batch, seqlen, dim, width, _ptr(u))
    if rc != 0:
        raise ValueError("oracle_conv1d_silu rejected its arguments")
    return u


def ssd(x: np.ndarray, dt: np.ndarray, A: np.ndarray, B: np.ndarray, C: np.ndarray,
        D: Optional[np.ndarray] = None, h0: Optional[np.ndarray] = None,
        heads: Optional[Sequence[int]] = None, threads: int = 1, _lib=None) -> Dict[str, np.ndarray]:
    """fp64 multi-head recurrence.  x (B, L, H, P), dt (B, L, H), B, C (B, L, N) in float32 or
    bf16 bits; A, D (H,) float32; h0 (B, H, N, P) any float.  Returns ``y`` (B, L, H, P) and
    ``h_last`` (B, H, N, P) -- or (n, L, P) / (n, N, P) for ``heads`` = flat b*H + h.
    ``threads`` > 1 splits the (b, h) pairs over threads (bit-identical results)."""
    lib = _lib or _load()
    dtp = _dtype_of(x)
    batch, seqlen, nh, hdim = x.shape
    dstate = B.shape[2]
    for name, arr, shp in (("dt", dt, (batch, seqlen, nh)), ("B", B, (batch, seqlen, dstate)),
                           ("C", C, (batch, seqlen, dstate))):
        if tuple(arr.shape) != shp or _dtype_of(arr) != dtp:
            raise ValueError("%s has shape %s dtype %s" % (name, arr.shape, arr.dtype))
    x, dt, B, C = _c(x), _c(dt), _c(B), _c(C)
    A = _c(A, np.float32)
    D = _c(D, np.float32)
    h0 = _c(h0, np.float64)
    sel = None if heads is None else np.ascontiguousarray(np.asarray(heads, dtype=np.int64))
    n = batch * nh if sel is None else sel.size
    y = np.empty((n, seqlen, hdim))
    hl = np.empty((n, dstate, hdim))
    rc = lib.oracle_ssd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), dtp, batch, seqlen, nh,
                        hdim, dstate, _ptr(sel), n, _ptr(y), _ptr(hl), int(threads))
    if rc != 0:
        raise ValueError("oracle_ssd rejected its arguments")
    if sel is None:
        return {"y": y.reshape(batch, nh, seqlen, hdim).transpose(0, 2, 1, 3).copy(),
                "h_last": hl.reshape(batch, nh, dstate, hdim)}
    return {"y": y, "h_last": hl}


def widen(a: np.ndarray) -> np.ndarray:
    """Exact float64 view of a float32 or bf16-bits operand."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


from .twin import twin_scan  # noqa: E402  (NumPy statement of the same definition)
