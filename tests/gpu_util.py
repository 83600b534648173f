"""Helpers shared by the GPU parity tests: host<->device moves and the error metric."""
from __future__ import annotations

import sys

import numpy as np
import torch

# max relative error bars (fp32 inputs; bf16 inputs with fp32 state)
TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(*msg) -> None:
    """Name the case on stdout before a GPU step (flushed, so it survives a crash)."""
    print(*msg, flush=True)
    sys.stdout.flush()


def dev(a, device="cuda"):
    """numpy (float32, or uint16 bf16 bits) -> device tensor (float32 / bfloat16)."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host64(t: torch.Tensor) -> np.ndarray:
    """device tensor -> float64 numpy (bf16 widened exactly)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).numpy().view(np.uint16)
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return t.double().numpy()


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max_i |got_i - ref_i| / max(|ref_i|, rms(ref)); the rms floor keeps outputs that
    cancel to ~0 from dominating."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    denom = np.maximum(np.abs(ref), rms)
    denom = np.where(denom == 0.0, 1.0, denom)
    return float(np.max(np.abs(got - ref) / denom))


def lanes_of(y_bld: np.ndarray, lanes) -> np.ndarray:
    """(B, L, D) -> (n_lanes, L) for flat lanes b*D + d."""
    nb, nl, nd = y_bld.shape
    lanes = np.asarray(lanes)
    return y_bld[lanes // nd, :, lanes % nd]


def sample_lanes(batch: int, dim: int, count: int, seed: int = 0) -> np.ndarray:
    """Lanes b*D+d covering both ends of every axis plus a seeded random spread."""
    rng = np.random.default_rng(seed)
    picks = {0, dim - 1, (batch - 1) * dim, batch * dim - 1}
    for d in (63, 64, dim // 2):
        if d < dim:
            picks.add(d)
            picks.add((batch - 1) * dim + d)
    while len(picks) < min(count, batch * dim):
        picks.add(int(rng.integers(0, batch * dim)))
    return np.array(sorted(picks), dtype=np.int64)
