"""Seeded synthetic inputs for the selective scan and the recurrent step.

This module is shared by the CPU oracle's tests, the GPU parity tests, the
bench and the smoke check.  It holds the workload table and the random
generators only: nothing of the scan itself (no discretisation, recurrence,
contraction or gating) is computed here.

Recipe (one place, so every consumer draws identical bits):

* Each tensor comes from its own PCG64 stream,
  ``numpy.random.default_rng([seed, cfg_id, tensor_id, step])``, so tensors can
  be drawn independently and in any order.
* Normals are drawn in float32.  The step size is the softplus of a normal,
  ``softplus(x) = log(1 + e^x)`` (the positivity map the Mamba pages put in
  front of the scan, Mamba walk-through section 3.1 and the LTI chapter
  section 0.4.2), evaluated in float32 with ``numpy.logaddexp``.
* bf16 tensors are rounded once from float32 with round-to-nearest-even and
  handed to both sides as raw 16-bit patterns (``numpy.uint16``).
* A is fp32 (D, N).  ``A[d, n] = -(n + 1)`` is the initialisation of the Mamba
  block (walk-through section 3.4); the "perturbed" recipe multiplies it by
  ``exp(U(-1/2, 1/2))`` per (d, n).  D (skip) is fp32 (D,), h0 fp32 (B, D, N).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, Iterator, Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"

# tensor ids for the per-tensor streams
_TID = {"u": 0, "delta": 1, "A": 2, "B": 3, "C": 4, "D": 5, "z": 6, "h0": 7, "delta_bias": 8,
        "x": 9, "dt": 10}

_CHUNK = 1 << 22  # values per generation block (bounds the float32 temporaries)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtype and value distributions."""

    name: str
    cfg_id: int
    batch: int
    seqlen: int  # 1 for the recurrent step
    dim: int
    dstate: int
    dtype: str  # dtype of u, delta, B, C, z and y
    delta_mu: float
    delta_sigma: float
    a_perturbed: bool  # A = -(n+1)*exp(U(-.5,.5)) instead of -(n+1)
    has_D: bool
    has_z: bool
    has_h0: bool = False
    steps: int = 0  # chained recurrent steps (0: full-sequence scan)
    note: str = field(default="", compare=False)

    @property
    def elements(self) -> int:
        """Scan elements B*L*D*N per call (per step for the recurrent step)."""
        return self.batch * self.seqlen * self.dim * self.dstate


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, 1, 256, 64, 16, F32, -1.0, 0.5, False, False, False,
                     note="tiny fp32 scan"),
    "small": Workload("small", 2, 2, 2048, 1536, 16, BF16, -2.0, 1.0, True, True, True,
                      note="small-model layer, d_inner 1536"),
    "large": Workload("large", 3, 8, 2048, 5120, 16, BF16, -2.0, 1.0, True, True, True,
                      note="large-model layer, d_inner 5120"),
    "long": Workload("long", 4, 1, 131072, 2048, 16, BF16, -3.0, 1.0, False, False, False,
                     note="long context, multi-chunk carries"),
    "step": Workload("step", 5, 256, 1, 5120, 16, BF16, -2.0, 1.0, True, True, True,
                     has_h0=True, steps=1000, note="recurrent decode step, 1000 chained"),
}


def _rng(seed: int, cfg_id: int, tensor: str, step: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, cfg_id, _TID[tensor], step])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); return uint16 bits.

    Inputs must be finite: the largest finite pattern plus the rounding bias
    still fits in 32 bits, so the arithmetic stays in uint32.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16 rounding expects finite values")
    bits = x.view(np.uint32)
    out = np.empty(bits.shape, dtype=np.uint16)
    flat_in = bits.reshape(-1)
    flat_out = out.reshape(-1)
    for s in range(0, flat_in.size, _CHUNK):
        b = flat_in[s:s + _CHUNK]
        bias = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
        flat_out[s:s + _CHUNK] = ((b + bias) >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, mu: float = 0.0, sigma: float = 1.0) -> np.ndarray:
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    for s in range(0, out.size, _CHUNK):
        n = min(_CHUNK, out.size - s)
        v = rng.standard_normal(n, dtype=np.float32)
        if sigma != 1.0:
            v *= np.float32(sigma)
        if mu != 0.0:
            v += np.float32(mu)
        out[s:s + n] = v
    return out.reshape(shape)


def _softplus_normal(rng: np.random.Generator, shape, mu: float, sigma: float) -> np.ndarray:
    v = _normal(rng, shape, mu, sigma).reshape(-1)
    for s in range(0, v.size, _CHUNK):
        x = v[s:s + _CHUNK]
        # log(1 + e^x) = max(x, 0) + log(1 + e^-|x|), no overflow for large |x|
        v[s:s + _CHUNK] = np.maximum(x, np.float32(0.0)) + np.log1p(np.exp(-np.abs(x)))
    return v.reshape(shape)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == BF16 else np.ascontiguousarray(x, dtype=np.float32)


def make_A(dim: int, dstate: int, perturbed: bool, seed: int = 0, cfg_id: int = 0) -> np.ndarray:
    """A (D, N) fp32: -(n+1), optionally times exp(U(-1/2, 1/2)) per entry."""
    base = -np.arange(1, dstate + 1, dtype=np.float64)[None, :].repeat(dim, axis=0)
    if perturbed:
        r = _rng(seed, cfg_id, "A").uniform(-0.5, 0.5, size=(dim, dstate))
        base = base * np.exp(r)
    return base.astype(np.float32)


def scan_inputs(batch: int, seqlen: int, dim: int, dstate: int, dtype: str = BF16, *,
                delta_mu: float = -2.0, delta_sigma: float = 1.0, a_perturbed: bool = True,
                has_D: bool = True, has_z: bool = True, has_h0: bool = False,
                seed: int = 0, cfg_id: int = 0) -> Dict[str, Optional[np.ndarray]]:
    """Full-sequence inputs: u, delta, z (B,L,D); B, C (B,L,N); A (D,N); D (D,); h0 (B,D,N).

    Stored dtypes: ``dtype`` for u/delta/B/C/z (uint16 bits for bf16), fp32 for A, D, h0.
    Absent optional tensors are ``None``.
    """
    shp_x = (batch, seqlen, dim)
    shp_s = (batch, seqlen, dstate)
    out: Dict[str, Optional[np.ndarray]] = {}
    out["u"] = _store(_normal(_rng(seed, cfg_id, "u"), shp_x), dtype)
    out["delta"] = _store(_softplus_normal(_rng(seed, cfg_id, "delta"), shp_x, delta_mu, delta_sigma), dtype)
    out["A"] = make_A(dim, dstate, a_perturbed, seed, cfg_id)
    out["B"] = _store(_normal(_rng(seed, cfg_id, "B"), shp_s), dtype)
    out["C"] = _store(_normal(_rng(seed, cfg_id, "C"), shp_s), dtype)
    out["D"] = _normal(_rng(seed, cfg_id, "D"), (dim,)) if has_D else None
    out["z"] = _store(_normal(_rng(seed, cfg_id, "z"), shp_x), dtype) if has_z else None
    out["h0"] = _normal(_rng(seed, cfg_id, "h0"), (batch, dim, dstate)) if has_h0 else None
    return out


def with_raw_delta(inp: Dict[str, Optional[np.ndarray]], *, raw_sigma: float = 0.5, dt_min: float = 1e-3,
                   dt_max: float = 1e-1, seed: int = 0, cfg_id: int = 0) -> Dict[str, Optional[np.ndarray]]:
    """Inputs for the softplus option: ``delta`` replaced by a raw pre-softplus value
    N(0, raw_sigma) of the same shape and dtype, plus ``delta_bias`` (D,) float32 whose
    softplus, log(1 + e^b), is a step size drawn log-uniformly from [dt_min, dt_max]
    (the bias is stored as its inverse, log(e^dt - 1))."""
    out = dict(inp)
    dtype = BF16 if inp["u"].dtype == np.uint16 else F32
    shp_x = inp["u"].shape
    out["delta"] = _store(_normal(_rng(seed, cfg_id, "delta", 1), shp_x, 0.0, raw_sigma), dtype)
    dim = shp_x[-1]
    g = _rng(seed, cfg_id, "delta_bias")
    dt = np.exp(g.uniform(np.log(dt_min), np.log(dt_max), dim))
    out["delta_bias"] = np.log(np.expm1(dt)).astype(np.float32)
    return out


def ssd_inputs(batch: int, seqlen: int, heads: int, hdim: int, dstate: int, *, has_D: bool = True,
               has_h0: bool = False, seed: int = 0, cfg_id: int = 0) -> Dict[str, Optional[np.ndarray]]:
    """Inputs of the multi-head recurrence, bf16 bits for x (B,L,H,P), dt (B,L,H), B and C
    (B,L,N); fp32 A (H,) = -U(1, 16), D (H,) ~ N(0,1), h0 (B,H,N,P) ~ N(0,1).
    dt = softplus(N(-2, 1)) as for the scan; x, B, C ~ N(0, 1)."""
    out: Dict[str, Optional[np.ndarray]] = {}
    out["x"] = _store(_normal(_rng(seed, cfg_id, "x"), (batch, seqlen, heads, hdim)), BF16)
    out["dt"] = _store(_softplus_normal(_rng(seed, cfg_id, "dt"), (batch, seqlen, heads), -2.0, 1.0), BF16)
    out["A"] = (-_rng(seed, cfg_id, "A").uniform(1.0, 16.0, heads)).astype(np.float32)
    out["B"] = _store(_normal(_rng(seed, cfg_id, "B"), (batch, seqlen, dstate)), BF16)
    out["C"] = _store(_normal(_rng(seed, cfg_id, "C"), (batch, seqlen, dstate)), BF16)
    out["D"] = _normal(_rng(seed, cfg_id, "D"), (heads,)) if has_D else None
    out["h0"] = _normal(_rng(seed, cfg_id, "h0"), (batch, heads, dstate, hdim)) if has_h0 else None
    return out


def algorithmic_bytes_ssd(batch: int, seqlen: int, heads: int, hdim: int, dstate: int, has_D: bool = True) -> int:
    """HBM bytes the multi-head recurrence must move: x read and y written (bf16), dt, B and C
    read (bf16), A and D (fp32)."""
    rows = batch * seqlen
    return 2 * 2 * rows * heads * hdim + 2 * rows * heads + 2 * 2 * rows * dstate + 4 * heads * (1 + int(has_D))


def workload_inputs(w: Workload, seed: int = 0) -> Dict[str, Optional[np.ndarray]]:
    """Inputs of a full-sequence workload (not the recurrent step)."""
    if w.steps:
        raise ValueError("use step_params/step_inputs for the recurrent-step workload")
    return scan_inputs(w.batch, w.seqlen, w.dim, w.dstate, w.dtype,
                       delta_mu=w.delta_mu, delta_sigma=w.delta_sigma,
                       a_perturbed=w.a_perturbed, has_D=w.has_D, has_z=w.has_z,
                       has_h0=w.has_h0, seed=seed, cfg_id=w.cfg_id)


def step_params(w: Workload, seed: int = 0) -> Dict[str, Optional[np.ndarray]]:
    """Per-layer tensors of the recurrent step: A (D,N), D (D,), initial state h0 (B,D,N)."""
    return {
        "A": make_A(w.dim, w.dstate, w.a_perturbed, seed, w.cfg_id),
        "D": _normal(_rng(seed, w.cfg_id, "D"), (w.dim,)) if w.has_D else None,
        "h0": _normal(_rng(seed, w.cfg_id, "h0"), (w.batch, w.dim, w.dstate)),
    }


def step_inputs(w: Workload, step: int, seed: int = 0) -> Dict[str, Optional[np.ndarray]]:
    """Fresh per-token inputs of chained step ``step``: u, delta, z (B,D); B, C (B,N)."""
    s = step + 1  # stream 0 is reserved for the per-layer tensors
    shp_x = (w.batch, w.dim)
    shp_s = (w.batch, w.dstate)
    return {
        "u": _store(_normal(_rng(seed, w.cfg_id, "u", s), shp_x), w.dtype),
        "delta": _store(_softplus_normal(_rng(seed, w.cfg_id, "delta", s), shp_x,
                                         w.delta_mu, w.delta_sigma), w.dtype),
        "B": _store(_normal(_rng(seed, w.cfg_id, "B", s), shp_s), w.dtype),
        "C": _store(_normal(_rng(seed, w.cfg_id, "C", s), shp_s), w.dtype),
        "z": _store(_normal(_rng(seed, w.cfg_id, "z", s), shp_x), w.dtype) if w.has_z else None,
    }


def iter_step_inputs(w: Workload, steps: int, seed: int = 0, workers: int = 1) -> Iterator[Dict]:
    """step_inputs(w, 0..steps-1) in order.  With workers > 1 the steps are drawn
    ahead by a thread pool (numpy releases the GIL while it fills arrays); each
    step has its own seeded streams, so the result does not depend on it."""
    if workers <= 1:
        for s in range(steps):
            yield step_inputs(w, s, seed)
        return
    with ThreadPoolExecutor(max_workers=workers) as ex:
        ahead = 2 * workers
        futs = [ex.submit(step_inputs, w, s, seed) for s in range(min(ahead, steps))]
        for s in range(steps):
            item = futs[s].result()
            futs[s] = None
            if s + ahead < steps:
                futs.append(ex.submit(step_inputs, w, s + ahead, seed))
            yield item


def algorithmic_bytes_scan(batch: int, seqlen: int, dim: int, dstate: int, dtype: str,
                           has_D: bool, has_z: bool, h0: bool = False, h_last: bool = False) -> int:
    """Bytes a fused scan must move: each (B,L,D) / (B,L,N) tensor once, y written once."""
    s = 2 if dtype == BF16 else 4
    rows = batch * seqlen * dim
    n_x = 2 + (1 if has_z else 0) + 1  # u, delta, [z] read; y written
    total = n_x * rows * s + 2 * batch * seqlen * dstate * s + 4 * dim * dstate
    total += 4 * dim if has_D else 0
    total += 4 * batch * dim * dstate * (int(h0) + int(h_last))
    return total


def algorithmic_bytes_step(batch: int, dim: int, dstate: int, dtype: str, has_D: bool, has_z: bool) -> int:
    """Bytes one recurrent step must move: h read and written, per-token operands once."""
    s = 2 if dtype == BF16 else 4
    n_x = 2 + (1 if has_z else 0) + 1
    total = 8 * batch * dim * dstate + n_x * batch * dim * s + 2 * batch * dstate * s + 4 * dim * dstate
    total += 4 * dim if has_D else 0
    return total
