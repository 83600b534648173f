"""Seeded random-shape parity sweep over every entry point, against the fp64 oracle.

The hand-picked cases in the other GPU tests cover the documented edges; this
sweep draws further shapes (batch, length and channel counts that are not
multiples of the tile, wave or chunk sizes), dtypes, optional tensors, options
and forced chunk lengths from a fixed seed, so every run checks the same cases.
Tolerances as everywhere: max relative error 1e-4 (fp32 inputs), 2e-2 (bf16).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import TOL, dev, host64, rel_err, say

pytestmark = pytest.mark.gpu

THREADS = min(16, os.cpu_count() or 1)


def ss():
    import selective_state_space_85_amd as m

    return m


def tol_of(dtype):
    return TOL["bf16" if dtype == wl.BF16 else "f32"]


def draw_scan_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        b = int(rng.integers(1, 4))
        l = int(rng.integers(1, 700))
        d = int(rng.integers(1, 300))
        dtype = wl.F32 if rng.random() < 0.5 else wl.BF16
        chunk = int(rng.choice([0, 0, 16, 37, 64, 128, 500]))
        sp, zoh = bool(rng.random() < 0.4), bool(rng.random() < 0.3)
        cases.append((i, b, l, d, dtype, chunk, bool(rng.random() < 0.7), bool(rng.random() < 0.7),
                      bool(rng.random() < 0.5), sp, zoh))
    return cases


SCAN_CASES = draw_scan_cases(16, 2024)


@pytest.mark.parametrize("case", SCAN_CASES, ids=["scan%02d-B%dL%dD%d-%s-T%d" % c[:6] for c in SCAN_CASES])
def test_random_scan(case):
    i, b, l, d, dtype, chunk, has_D, has_z, has_h0, sp, zoh = case
    inp = wl.scan_inputs(b, l, d, 16, dtype, has_D=has_D, has_z=has_z, has_h0=has_h0, seed=300 + i)
    if sp:
        inp = wl.with_raw_delta(inp, seed=300 + i)
    m = ss()
    t = {k: dev(v) for k, v in inp.items()}
    say("random scan %d: B%d L%d D%d %s T=%d D=%s z=%s h0=%s softplus=%s zoh=%s" % case)
    y, hl = m.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t.get("D"), z=t.get("z"), h0=t.get("h0"),
                       delta_bias=t.get("delta_bias"), delta_softplus=sp, zoh=zoh, return_last_state=True,
                       chunk_len=chunk)
    torch.cuda.synchronize()
    ref = oracle.scan(**inp, delta_softplus=sp, zoh=zoh, threads=THREADS)
    ey, eh = rel_err(host64(y), ref["y"]), rel_err(host64(hl), ref["h_last"])
    say("  y err %.3e, h_last err %.3e" % (ey, eh))
    assert ey <= tol_of(dtype) and eh <= tol_of(dtype)


def draw_bwd_cases(n, seed):
    rng = np.random.default_rng(seed)
    return [(i, int(rng.integers(1, 3)), int(rng.integers(1, 200)), int(rng.integers(1, 150)),
             wl.F32 if rng.random() < 0.6 else wl.BF16, bool(rng.random() < 0.7), bool(rng.random() < 0.7),
             bool(rng.random() < 0.5), bool(rng.random() < 0.4)) for i in range(n)]


BWD_CASES = draw_bwd_cases(10, 2025)


@pytest.mark.parametrize("case", BWD_CASES, ids=["bwd%02d-B%dL%dD%d-%s" % c[:5] for c in BWD_CASES])
def test_random_bwd(case):
    i, b, l, d, dtype, has_D, has_z, has_h0, sp = case
    zoh = i % 4 in (1, 2)  # half of the cases under the zero-order-hold input term
    inp = wl.scan_inputs(b, l, d, 16, dtype, has_D=has_D, has_z=has_z, has_h0=has_h0, seed=400 + i)
    if sp:
        inp = wl.with_raw_delta(inp, seed=400 + i)
    rng = np.random.default_rng(500 + i)
    dy = rng.standard_normal((b, l, d)).astype(np.float32)
    if dtype == wl.BF16:
        dy = wl.f32_to_bf16_bits(dy)
    dhl = rng.standard_normal((b, d, 16)).astype(np.float32)
    t = {k: dev(v) for k, v in inp.items()}
    say("random bwd %d: B%d L%d D%d %s D=%s z=%s h0=%s softplus=%s" % case + " zoh=%s" % zoh)
    g = ss().scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dev(dy), D=t.get("D"), z=t.get("z"),
                      h0=t.get("h0"), dh_last=dev(dhl), delta_bias=t.get("delta_bias"), delta_softplus=sp, zoh=zoh)
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(**inp, dy=oracle.widen(dy), dh_last=dhl, delta_softplus=sp, zoh=zoh, threads=THREADS)
    for k, r in ref.items():
        e = rel_err(host64(g[k]), r)
        assert e <= tol_of(dtype), "%s: %.3e" % (k, e)


def test_random_conv_and_step():
    rng = np.random.default_rng(2026)
    m = ss()
    for i in range(6):
        b, l, d, width = int(rng.integers(1, 4)), int(rng.integers(1, 300)), int(rng.integers(1, 400)), \
            int(rng.integers(2, 5))
        stride = d + int(rng.integers(0, 3)) * d
        dtype = wl.F32 if i % 2 else wl.BF16
        x = rng.standard_normal((b, l, stride)).astype(np.float32)
        if dtype == wl.BF16:
            x = wl.f32_to_bf16_bits(x)
        w = (rng.standard_normal((d, width)) * 0.5).astype(np.float32)
        bias = rng.standard_normal(d).astype(np.float32) if i % 3 else None
        say("random conv %d: B%d L%d D%d stride %d width %d %s" % (i, b, l, d, stride, width, dtype))
        u = m.conv1d_silu(dev(x)[..., :d], dev(w), dev(bias))
        torch.cuda.synchronize()
        assert rel_err(host64(u), oracle.conv1d_silu(x, w, bias, dim=d)) <= tol_of(dtype)

        # a few chained steps of a random-size state
        inp = wl.scan_inputs(b, 3, d, 16, dtype, has_D=bool(i % 2), has_z=bool(i % 3), has_h0=True, seed=600 + i)
        t = {k: dev(v) for k, v in inp.items()}
        h = t["h0"].clone()
        href = inp["h0"].astype(np.float64).copy()
        for s in range(3):
            col = lambda v: None if v is None else np.ascontiguousarray(v[:, s])  # noqa: E731
            ys = m.step(h, t["u"][:, s].contiguous(), t["delta"][:, s].contiguous(), t["A"],
                        t["B"][:, s].contiguous(), t["C"][:, s].contiguous(), D=t.get("D"),
                        z=None if t.get("z") is None else t["z"][:, s].contiguous())
            yref = oracle.step(href, col(inp["u"]), col(inp["delta"]), inp["A"], col(inp["B"]), col(inp["C"]),
                               D=inp.get("D"), z=col(inp.get("z")))
            torch.cuda.synchronize()
            assert rel_err(host64(ys), yref) <= tol_of(dtype)
        assert rel_err(host64(h), href) <= tol_of(dtype)


def test_random_ssd():
    rng = np.random.default_rng(2027)
    m = ss()
    for i in range(8):
        b, l, h, n = int(rng.integers(1, 3)), int(rng.integers(1, 400)), int(rng.integers(1, 5)), \
            int(rng.choice([64, 128, 256]))
        has_D, has_h0 = bool(i % 2), bool(i % 3)
        inp = wl.ssd_inputs(b, l, h, 64, n, has_D=has_D, has_h0=has_h0, seed=700 + i)
        t = {k: dev(v) for k, v in inp.items()}
        say("random ssd %d: B%d L%d H%d N%d D=%s h0=%s" % (i, b, l, h, n, has_D, has_h0))
        y, hl = m.ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t.get("D"), h0=t.get("h0"),
                          return_last_state=True)
        torch.cuda.synchronize()
        ref = oracle.ssd(**inp)
        assert rel_err(host64(y), ref["y"]) <= TOL["bf16"]
        assert rel_err(host64(hl), ref["h_last"]) <= TOL["bf16"]
