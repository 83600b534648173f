"""torch-facing wrappers of the C ABI: argument marshalling only.

Every step of the scan runs in the HIP kernels of libssscan.so; torch supplies
device memory and the current stream.  Names and argument order follow the
C entry points (``ss_scan_fwd`` -> ``scan_fwd``, ``ss_step`` -> ``step``).
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional, Tuple, Union

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.SS_F32, torch.bfloat16: _lib.SS_BF16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, shape, dtype, device) -> None:
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def scan_plan(batch: int, seqlen: int, dim: int, dstate: int, chunk_len: int = 0) -> Tuple[int, int]:
    """(chunk_len, n_chunks) that ``ss_scan_fwd`` uses for this shape (``ss_scan_plan``), or,
    with a ``chunk_len`` request, ``ss_scan_fwd_ex`` (``ss_scan_plan_ex``)."""
    T = ctypes.c_int64()
    K = ctypes.c_int64()
    lib = _lib.load()
    if chunk_len == 0:
        _lib.check("ss_scan_plan", lib.ss_scan_plan(batch, seqlen, dim, dstate, ctypes.byref(T), ctypes.byref(K)))
    else:
        _lib.check("ss_scan_plan_ex", lib.ss_scan_plan_ex(batch, seqlen, dim, dstate, chunk_len,
                                                          ctypes.byref(T), ctypes.byref(K)))
    return T.value, K.value


def _options(delta_softplus: bool, zoh: bool) -> int:
    return (_lib.SS_DELTA_SOFTPLUS if delta_softplus else 0) | (_lib.SS_B_ZOH if zoh else 0)


def scan_workspace_bytes(batch: int, seqlen: int, dim: int, dstate: int, chunk_len: int = 0) -> int:
    """Workspace bytes of ``ss_scan_fwd`` (``ss_scan_workspace_bytes``), or for a ``chunk_len``
    request ``ss_scan_workspace_bytes_ex``."""
    lib = _lib.load()
    if chunk_len == 0:
        n = lib.ss_scan_workspace_bytes(batch, seqlen, dim, dstate)
    else:
        n = lib.ss_scan_workspace_bytes_ex(batch, seqlen, dim, dstate, chunk_len)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid scan shape")
    return int(n)


def scan_fwd(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
             D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
             h0: Optional[torch.Tensor] = None, *, return_last_state: bool = False,
             chunk_len: int = 0, out: Optional[torch.Tensor] = None,
             h_last: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
             delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = False, zoh: bool = False,
             ckpt: Optional[torch.Tensor] = None) -> Union[torch.Tensor, Tuple[torch.Tensor, torch.Tensor]]:
    """Selective scan on device tensors: ``ss_scan_fwd``, or ``ss_scan_fwd_ex`` when a step-size
    or input-term option or a ``chunk_len`` request is given; with ``ckpt`` (a float32 tensor of
    ``scan_ckpt_shape(B, L, D, N)``) it is ``ss_scan_fwd_ckpt``, which also writes there the
    state entering every 16th timestep for ``scan_bwd(..., ckpt=ckpt)``.

    u, delta, z: (B, L, D); B, C: (B, L, N) -- all float32 or all bfloat16.
    A: (D, N) float32; D: (D,) float32; h0: (B, D, N) float32.
    delta_bias (D,) float32 / delta_softplus: step size softplus(delta + bias[d]);
    zoh: zero-order-hold input term instead of Euler's delta*B.
    Returns y (B, L, D) in the input dtype, and h_last (B, D, N) float32 if asked.
    ``out`` / ``h_last`` / ``workspace`` may be passed in to avoid allocation.
    """
    if u.dim() != 3:
        raise ValueError("u must be (batch, seqlen, dim)")
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("scan_fwd runs on the GPU; u is on %s" % dev)
    dt = u.dtype
    if dt not in _DTYPES:
        raise TypeError("unsupported dtype %s" % dt)
    nb, nl, nd = u.shape
    nn = A.shape[-1]
    _need(u, "u", (nb, nl, nd), dt, dev)
    _need(delta, "delta", (nb, nl, nd), dt, dev)
    _need(A, "A", (nd, nn), torch.float32, dev)
    _need(B, "B", (nb, nl, nn), dt, dev)
    _need(C, "C", (nb, nl, nn), dt, dev)
    if D is not None:
        _need(D, "D", (nd,), torch.float32, dev)
    if z is not None:
        _need(z, "z", (nb, nl, nd), dt, dev)
    if h0 is not None:
        _need(h0, "h0", (nb, nd, nn), torch.float32, dev)
    if delta_bias is not None:
        _need(delta_bias, "delta_bias", (nd,), torch.float32, dev)
    y = out if out is not None else torch.empty((nb, nl, nd), dtype=dt, device=dev)
    _need(y, "out", (nb, nl, nd), dt, dev)
    hl = h_last
    if return_last_state and hl is None:
        hl = torch.empty((nb, nd, nn), dtype=torch.float32, device=dev)
    if hl is not None:
        _need(hl, "h_last", (nb, nd, nn), torch.float32, dev)
    if ckpt is not None:
        _need(ckpt, "ckpt", scan_ckpt_shape(nb, nl, nd, nn), torch.float32, dev)
    need = scan_workspace_bytes(nb, nl, nd, nn, chunk_len)
    ws = workspace
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    lib = _lib.load()
    with torch.cuda.device(dev):
        if ckpt is None and delta_bias is None and not delta_softplus and not zoh and chunk_len == 0:
            name = "ss_scan_fwd"
            st = lib.ss_scan_fwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                 _ptr(y), _ptr(hl), _ptr(ws), ws_bytes, nb, nl, nd, nn, _DTYPES[dt], _stream(dev))
        elif ckpt is None:
            name = "ss_scan_fwd_ex"
            st = lib.ss_scan_fwd_ex(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                    _ptr(delta_bias), _options(delta_softplus, zoh), _ptr(y), _ptr(hl),
                                    _ptr(ws), ws_bytes, nb, nl, nd, nn, chunk_len, _DTYPES[dt], _stream(dev))
        else:
            name = "ss_scan_fwd_ckpt"
            st = lib.ss_scan_fwd_ckpt(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                      _ptr(h0), _ptr(delta_bias), _options(delta_softplus, zoh), _ptr(y), _ptr(hl),
                                      _ptr(ckpt), _ptr(ws), ws_bytes, nb, nl, nd, nn, chunk_len, _DTYPES[dt],
                                      _stream(dev))
    _lib.check(name, st)
    if return_last_state:
        return y, hl
    return y


def scan_fwd_noalloc(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                     D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                     h0: Optional[torch.Tensor] = None, *, out: torch.Tensor,
                     h_last: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``ss_scan_fwd_noalloc``: the scan with the library's static per-GPU workspace, for
    callers that cannot allocate device memory.  ``out`` (and ``h_last`` if wanted) are the
    caller's; nothing is allocated here or in the library.  Shapes as for ``scan_fwd``; a
    shape whose workspace exceeds ``_lib.SS_NOALLOC_MAX_WORKSPACE_BYTES`` raises SSError.
    Calls that overlap in time on one GPU share that workspace and must not overlap."""
    if u.dim() != 3:
        raise ValueError("u must be (batch, seqlen, dim)")
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("scan_fwd_noalloc runs on the GPU; u is on %s" % dev)
    dt = u.dtype
    if dt not in _DTYPES:
        raise TypeError("unsupported dtype %s" % dt)
    nb, nl, nd = u.shape
    nn = A.shape[-1]
    for t, name, shp, tdt in ((u, "u", (nb, nl, nd), dt), (delta, "delta", (nb, nl, nd), dt),
                              (A, "A", (nd, nn), torch.float32), (B, "B", (nb, nl, nn), dt),
                              (C, "C", (nb, nl, nn), dt), (out, "out", (nb, nl, nd), dt)):
        _need(t, name, shp, tdt, dev)
    for t, name, shp, tdt in ((D, "D", (nd,), torch.float32), (z, "z", (nb, nl, nd), dt),
                              (h0, "h0", (nb, nd, nn), torch.float32), (h_last, "h_last", (nb, nd, nn), torch.float32)):
        if t is not None:
            _need(t, name, shp, tdt, dev)
    with torch.cuda.device(dev):
        st = _lib.load().ss_scan_fwd_noalloc(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                             _ptr(h0), _ptr(out), _ptr(h_last), nb, nl, nd, nn, _DTYPES[dt],
                                             _stream(dev))
    _lib.check("ss_scan_fwd_noalloc", st)
    return out


def step(h: torch.Tensor, u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
         C: torch.Tensor, D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
         *, out: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
         delta_softplus: bool = False, zoh: bool = False) -> torch.Tensor:
    """One recurrent token ``ss_step_ex``: h (B, D, N) float32 is updated in place.

    u, delta, z: (B, D); B, C: (B, N), float32 or bfloat16; A (D, N), D (D,) float32.
    delta_bias / delta_softplus / zoh as for ``scan_fwd``.
    Returns y (B, D) in the input dtype.
    """
    if u.dim() != 2:
        raise ValueError("u must be (batch, dim)")
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("step runs on the GPU; u is on %s" % dev)
    dt = u.dtype
    if dt not in _DTYPES:
        raise TypeError("unsupported dtype %s" % dt)
    nb, nd = u.shape
    nn = A.shape[-1]
    _need(h, "h", (nb, nd, nn), torch.float32, dev)
    _need(delta, "delta", (nb, nd), dt, dev)
    _need(A, "A", (nd, nn), torch.float32, dev)
    _need(B, "B", (nb, nn), dt, dev)
    _need(C, "C", (nb, nn), dt, dev)
    if D is not None:
        _need(D, "D", (nd,), torch.float32, dev)
    if z is not None:
        _need(z, "z", (nb, nd), dt, dev)
    if delta_bias is not None:
        _need(delta_bias, "delta_bias", (nd,), torch.float32, dev)
    y = out if out is not None else torch.empty((nb, nd), dtype=dt, device=dev)
    _need(y, "out", (nb, nd), dt, dev)
    with torch.cuda.device(dev):
        st = _lib.load().ss_step_ex(_ptr(h), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                    _ptr(z), _ptr(delta_bias), _options(delta_softplus, zoh), _ptr(y),
                                    nb, nd, nn, _DTYPES[dt], _stream(dev))
    _lib.check("ss_step_ex", st)
    return y


def scan_ckpt_shape(batch: int, seqlen: int, dim: int, dstate: int) -> Tuple[int, int, int, int]:
    """Shape of the float32 state checkpoints (``ss_scan_ckpt_bytes``): one state every 16
    timesteps, laid out (ceil(L/16), B, N, D)."""
    n = _lib.load().ss_scan_ckpt_bytes(batch, seqlen, dim, dstate)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid scan shape")
    return (-(-seqlen // 16), batch, dstate, dim)


def scan_bwd_workspace_bytes(batch: int, seqlen: int, dim: int, dstate: int, with_ckpt: bool = False) -> int:
    """Workspace of ``ss_scan_bwd`` (or, with_ckpt, of ``ss_scan_bwd_ckpt``)."""
    lib = _lib.load()
    fn = lib.ss_scan_bwd_ckpt_workspace_bytes if with_ckpt else lib.ss_scan_bwd_workspace_bytes
    n = fn(batch, seqlen, dim, dstate)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid scan shape")
    return int(n)


def scan_bwd(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
             dy: torch.Tensor, D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
             h0: Optional[torch.Tensor] = None, *, dh_last: Optional[torch.Tensor] = None,
             delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = False, zoh: bool = False,
             want_dh0: bool = True, workspace: Optional[torch.Tensor] = None,
             ckpt: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Gradients of sum(dy * y) + sum(dh_last * h_last) for ``scan_fwd`` with the same inputs
    and options (``ss_scan_bwd``).  dy (B, L, D) in the input dtype; dh_last (B, D, N) float32 or None.
    With ``ckpt`` (the checkpoints ``scan_fwd(..., ckpt=ckpt)`` wrote) it is ``ss_scan_bwd_ckpt``,
    which reuses them instead of recomputing the states' checkpoints.

    Returns a dict: du, ddelta, dz (B, L, D) and dB, dC (B, L, N) in the input dtype; dA (D, N),
    dD (D,), ddelta_bias (D,), dh0 (B, D, N) float32.  Gradients of absent inputs are absent;
    dh0 only if ``want_dh0``.  ddelta is with respect to delta as passed (raw under softplus).
    """
    if u.dim() != 3:
        raise ValueError("u must be (batch, seqlen, dim)")
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("scan_bwd runs on the GPU; u is on %s" % dev)
    dt = u.dtype
    if dt not in _DTYPES:
        raise TypeError("unsupported dtype %s" % dt)
    nb, nl, nd = u.shape
    nn = A.shape[-1]
    for t, name, shp, tdt in ((u, "u", (nb, nl, nd), dt), (delta, "delta", (nb, nl, nd), dt),
                              (A, "A", (nd, nn), torch.float32), (B, "B", (nb, nl, nn), dt),
                              (C, "C", (nb, nl, nn), dt), (dy, "dy", (nb, nl, nd), dt)):
        _need(t, name, shp, tdt, dev)
    for t, name, shp, tdt in ((D, "D", (nd,), torch.float32), (z, "z", (nb, nl, nd), dt),
                              (h0, "h0", (nb, nd, nn), torch.float32),
                              (dh_last, "dh_last", (nb, nd, nn), torch.float32),
                              (delta_bias, "delta_bias", (nd,), torch.float32)):
        if t is not None:
            _need(t, name, shp, tdt, dev)
    g = {"du": torch.empty((nb, nl, nd), dtype=dt, device=dev),
         "ddelta": torch.empty((nb, nl, nd), dtype=dt, device=dev),
         "dA": torch.empty((nd, nn), dtype=torch.float32, device=dev),
         "dB": torch.empty((nb, nl, nn), dtype=dt, device=dev),
         "dC": torch.empty((nb, nl, nn), dtype=dt, device=dev)}
    if D is not None:
        g["dD"] = torch.empty((nd,), dtype=torch.float32, device=dev)
    if z is not None:
        g["dz"] = torch.empty((nb, nl, nd), dtype=dt, device=dev)
    if delta_bias is not None:
        g["ddelta_bias"] = torch.empty((nd,), dtype=torch.float32, device=dev)
    if want_dh0:
        g["dh0"] = torch.empty((nb, nd, nn), dtype=torch.float32, device=dev)
    if ckpt is not None:
        _need(ckpt, "ckpt", scan_ckpt_shape(nb, nl, nd, nn), torch.float32, dev)
    need = scan_bwd_workspace_bytes(nb, nl, nd, nn, with_ckpt=ckpt is not None)
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = ws.numel() * ws.element_size()
    opts = _options(delta_softplus, zoh)
    grads = (_ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g.get("dD")),
             _ptr(g.get("dz")), _ptr(g.get("ddelta_bias")), _ptr(g.get("dh0")))
    lib = _lib.load()
    with torch.cuda.device(dev):
        if ckpt is None:
            name = "ss_scan_bwd"
            st = lib.ss_scan_bwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                 _ptr(delta_bias), opts, _ptr(dy), _ptr(dh_last), *grads, _ptr(ws), ws_bytes,
                                 nb, nl, nd, nn, _DTYPES[dt], _stream(dev))
        else:
            name = "ss_scan_bwd_ckpt"
            st = lib.ss_scan_bwd_ckpt(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                      _ptr(delta_bias), opts, _ptr(dy), _ptr(dh_last), _ptr(ckpt), *grads,
                                      _ptr(ws), ws_bytes, nb, nl, nd, nn, _DTYPES[dt], _stream(dev))
    _lib.check(name, st)
    return g


def conv1d_silu(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None, *,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal depthwise convolution + SiLU ``ss_conv1d_silu``: u (B, L, D) from x (B, L, D),
    weight (D, width) float32, bias (D,) float32.  x may be a column slice with unit inner
    stride, e.g. ``xz[..., :D]`` of a contiguous (B, L, 2D) projection, read in place."""
    if x.dim() != 3:
        raise ValueError("x must be (batch, seqlen, dim)")
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("conv1d_silu runs on the GPU; x is on %s" % dev)
    dt = x.dtype
    if dt not in _DTYPES:
        raise TypeError("unsupported dtype %s" % dt)
    nb, nl, nd = x.shape
    if x.stride(2) != 1 or x.stride(0) != nl * x.stride(1):
        raise ValueError("x rows must be evenly strided with unit channel stride")
    if weight.dim() != 2 or weight.shape[0] != nd:
        raise ValueError("weight must be (dim, width)")
    _need(weight, "weight", tuple(weight.shape), torch.float32, dev)
    if bias is not None:
        _need(bias, "bias", (nd,), torch.float32, dev)
    u = out if out is not None else torch.empty((nb, nl, nd), dtype=dt, device=dev)
    _need(u, "out", (nb, nl, nd), dt, dev)
    with torch.cuda.device(dev):
        st = _lib.load().ss_conv1d_silu(_ptr(x), x.stride(1), _ptr(weight), _ptr(bias), _ptr(u), nb, nl, nd,
                                        weight.shape[1], _DTYPES[dt], _stream(dev))
    _lib.check("ss_conv1d_silu", st)
    return u


def ssd_fwd(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
            D: Optional[torch.Tensor] = None, h0: Optional[torch.Tensor] = None, *,
            return_last_state: bool = False, out: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None) -> Union[torch.Tensor, Tuple[torch.Tensor, torch.Tensor]]:
    """Multi-head state-space recurrence ``ss_ssd_fwd_ex`` (bf16, 64 channels per head).

    x (B, L, H, 64), dt (B, L, H), B and C (B, L, N) bfloat16 with N 64, 128 or 256; A, D (H,)
    float32; h0 (B, H, N, 64) float32.  Returns y (B, L, H, 64) bfloat16 and, if asked,
    h_last (B, H, N, 64) float32.  N = 256 needs ``ssd_workspace_bytes`` of workspace,
    allocated here when not passed."""
    if x.dim() != 4:
        raise ValueError("x must be (batch, seqlen, heads, headdim)")
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("ssd_fwd runs on the GPU; x is on %s" % dev)
    nb, nl, nh, hp = x.shape
    ns = B.shape[-1]
    dt_ = x.dtype
    for t, name, shp, tdt in ((x, "x", (nb, nl, nh, hp), dt_), (dt, "dt", (nb, nl, nh), dt_),
                              (A, "A", (nh,), torch.float32), (B, "B", (nb, nl, ns), dt_),
                              (C, "C", (nb, nl, ns), dt_)):
        _need(t, name, shp, tdt, dev)
    if D is not None:
        _need(D, "D", (nh,), torch.float32, dev)
    if h0 is not None:
        _need(h0, "h0", (nb, nh, ns, hp), torch.float32, dev)
    y = out if out is not None else torch.empty_like(x)
    _need(y, "out", (nb, nl, nh, hp), dt_, dev)
    hl = torch.empty((nb, nh, ns, hp), dtype=torch.float32, device=dev) if return_last_state else None
    need = ssd_workspace_bytes(nb, nl, nh, hp, ns)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        st = _lib.load().ss_ssd_fwd_ex(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(y),
                                       _ptr(hl), _ptr(workspace), ws_bytes, nb, nl, nh, hp, ns,
                                       _DTYPES.get(dt_, 99), _stream(dev))
    _lib.check("ss_ssd_fwd_ex", st)
    return (y, hl) if return_last_state else y


def ssd_workspace_bytes(batch: int, seqlen: int, heads: int, headdim: int, dstate: int) -> int:
    """Workspace of ``ss_ssd_fwd_ex`` (0 unless dstate is 256)."""
    n = _lib.load().ss_ssd_workspace_bytes(batch, seqlen, heads, headdim, dstate)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid multi-head recurrence shape")
    return int(n)
