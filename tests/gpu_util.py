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
    cancel to ~0 from dominating.  Large arrays are taken in blocks, so the temporaries
    stay small next to the operands."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    g = got.reshape(-1)
    r = ref.reshape(-1)
    blk = 1 << 24
    sq = 0.0
    for i in range(0, r.size, blk):
        rb = r[i:i + blk].astype(np.float64, copy=False)
        sq += float(np.dot(rb, rb))
    rms = float(np.sqrt(sq / r.size))
    worst = 0.0
    for i in range(0, r.size, blk):
        rb = r[i:i + blk].astype(np.float64, copy=False)
        gb = g[i:i + blk].astype(np.float64, copy=False)
        denom = np.maximum(np.abs(rb), rms)
        denom[denom == 0.0] = 1.0
        e = np.abs(gb - rb) / denom
        if np.isnan(e).any():
            return float("nan")
        worst = max(worst, float(e.max()))
    return worst
