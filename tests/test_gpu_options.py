"""GPU parity of the step-size and input-term options (ss_scan_fwd_ex / ss_step_ex)
against the fp64 CPU oracle:

* step size softplus(delta + bias[d]) (LTI chapter, section 3.1.4.2), and a bias
  added without softplus;
* the zero-order-hold input term (Mamba walk-through, section 2.2) instead of
  Euler's delta*B.

Same tolerances as the plain scan: max relative error <= 1e-4 for fp32 inputs,
<= 2e-2 for bf16 inputs with fp32 state.
"""
import os

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import TOL, dev, host64, rel_err, say

pytestmark = pytest.mark.gpu

THREADS = min(16, os.cpu_count() or 1)

# name -> options; "softplus" modes take a raw (pre-softplus) delta and a bias
MODES = {
    "softplus+bias": dict(delta_softplus=True),
    "zoh": dict(zoh=True),
    "softplus+bias+zoh": dict(delta_softplus=True, zoh=True),
    "bias": dict(),
}


def ss():
    import selective_state_space_85_amd as m

    return m


def make_case(mode, batch, seqlen, dim, dtype, seed):
    inp = wl.scan_inputs(batch, seqlen, dim, 16, dtype, has_D=True, has_z=True, has_h0=True, seed=seed)
    if "softplus" in mode:
        inp = wl.with_raw_delta(inp, seed=seed)
    elif mode == "bias":
        inp["delta_bias"] = np.random.default_rng(seed).uniform(0.0, 0.05, dim).astype(np.float32)
    return inp, MODES[mode]


def gpu_scan(inp, opts, chunk_len=0):
    t = {k: dev(v) for k, v in inp.items()}
    y, hl = ss().scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t.get("D"), z=t.get("z"),
                          h0=t.get("h0"), return_last_state=True, chunk_len=chunk_len,
                          delta_bias=t.get("delta_bias"), **opts)
    return host64(y), host64(hl)


def check(what, inp, y, hl, ref):
    tol = TOL["bf16" if inp["u"].dtype == np.uint16 else "f32"]
    ey = rel_err(y, ref["y"])
    eh = rel_err(hl, ref["h_last"])
    say("  %s: y err %.3e, h_last err %.3e (tol %.0e)" % (what, ey, eh, tol))
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(hl)), what
    assert ey <= tol and eh <= tol, what


@pytest.mark.parametrize("mode", list(MODES))
def test_options_fp32_plans(mode):
    """fp32, one and several chunks (the aggregate and carry passes see the same
    options), a few A = 0 entries (ZOH takes its Euler limit there) and, without
    softplus, rows with delta = 0 (state kept)."""
    inp, opts = make_case(mode, 1, 256, 64, wl.F32, seed=31)
    inp["A"] = inp["A"].copy()
    inp["A"][0, :4] = 0.0
    inp["A"][17, 5] = 0.0
    if "softplus" not in mode:
        inp["delta"] = inp["delta"].copy()
        inp["delta"][:, 5, :] = 0.0
        inp["delta"][:, 100:103, :7] = 0.0
    ref = oracle.scan(**inp, **opts)
    for T in (0, 64, 100):
        say("options %s fp32, chunk_len=%d" % (mode, T))
        y, hl = gpu_scan(inp, opts, chunk_len=T)
        check("%s T=%d" % (mode, T), inp, y.reshape(1, 256, 64), hl, ref)


@pytest.mark.parametrize("mode", list(MODES))
def test_options_bf16_ragged(mode):
    """bf16, a ragged channel tail (160 = 2.5 x 64) and a ragged last tile (600 rows)."""
    inp, opts = make_case(mode, 2, 600, 160, wl.BF16, seed=32)
    ref = oracle.scan(**inp, **opts, threads=THREADS)
    for T in (0, 64):
        say("options %s bf16 B2 L600 D160, chunk_len=%d" % (mode, T))
        y, hl = gpu_scan(inp, opts, chunk_len=T)
        check("%s T=%d" % (mode, T), inp, y, hl, ref)


def test_options_large_layer_full():
    """The large-layer shape (B8 L2048 D5120, bf16) with softplus + bias + ZOH, in the
    launch configuration of the plain bench (single chunk), every output element."""
    w = wl.WORKLOADS["large"]
    inp = wl.with_raw_delta(wl.workload_inputs(w), seed=0, cfg_id=w.cfg_id)
    opts = dict(delta_softplus=True, zoh=True)
    say("options softplus+bias+zoh on the large layer")
    y, hl = gpu_scan(inp, opts)
    assert np.all(np.isfinite(y))
    ref = oracle.scan(**inp, **opts, threads=THREADS)
    ey = rel_err(y, ref["y"])
    eh = rel_err(hl, ref["h_last"])
    say("  large with options: y err %.3e, h_last err %.3e, every lane" % (ey, eh))
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_options_step_chain(dtype):
    """40 chained ss_step_ex tokens with softplus + bias + ZOH against the oracle's
    step, and against one ss_scan_fwd_ex over the same tokens."""
    import torch

    m = ss()
    nb, nl, nd = 3, 40, 192
    inp, opts = make_case("softplus+bias+zoh", nb, nl, nd, dtype, seed=34)
    t = {k: dev(v) for k, v in inp.items()}
    say("options step chain (%s)" % dtype)
    h = t["h0"].clone()
    href = inp["h0"].astype(np.float64).copy()
    ys, yrefs = [], []
    for s in range(nl):
        col = lambda k: t[k][:, s].contiguous()  # noqa: E731
        ys.append(m.step(h, col("u"), col("delta"), t["A"], col("B"), col("C"), D=t["D"], z=col("z"),
                         delta_bias=t["delta_bias"], **opts))
        yrefs.append(oracle.step(href, inp["u"][:, s], inp["delta"][:, s], inp["A"], inp["B"][:, s],
                                 inp["C"][:, s], D=inp["D"], z=inp["z"][:, s], delta_bias=inp["delta_bias"],
                                 **opts))
    torch.cuda.synchronize()
    tol = TOL["bf16" if dtype == wl.BF16 else "f32"]
    y_steps = np.stack([host64(v) for v in ys], axis=1)
    ey = rel_err(y_steps, np.stack(yrefs, axis=1))
    eh = rel_err(host64(h), href)
    say("  step chain: y err %.3e, h err %.3e" % (ey, eh))
    assert ey <= tol and eh <= tol
    y_scan, h_scan = gpu_scan(inp, opts)
    assert rel_err(y_steps, y_scan) <= tol and rel_err(host64(h), h_scan) <= tol
