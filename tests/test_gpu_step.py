"""GPU parity of ss_step (single-token recurrent update) against the fp64 CPU oracle."""
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


def test_step_chain_1000():
    """The recurrent-step workload: B=256, D=5120, N=16, 1000 chained tokens; every lane's y at
    every token, and every lane's state every 250 tokens and at the end."""
    w = wl.WORKLOADS["step"]
    m = ss()
    p = wl.step_params(w)
    A_t, D_t = dev(p["A"]), dev(p["D"])
    h = dev(p["h0"]).clone()
    h_ref = p["h0"].astype(np.float64).copy()
    worst = 0.0
    say("step chain: %d steps, B=%d D=%d, every lane" % (w.steps, w.batch, w.dim))
    for s, inp in enumerate(wl.iter_step_inputs(w, w.steps, workers=8)):
        t = {k: dev(v) for k, v in inp.items()}
        y = m.step(h, t["u"], t["delta"], A_t, t["B"], t["C"], D=D_t, z=t["z"])
        y_ref = oracle.step(h_ref, inp["u"], inp["delta"], p["A"], inp["B"], inp["C"], D=p["D"],
                            z=inp["z"], threads=THREADS)
        e = rel_err(host64(y), y_ref)
        worst = max(worst, e)
        if s % 250 == 0 or s == w.steps - 1:
            eh = rel_err(host64(h), h_ref)
            say("  step %d: y err %.3e (worst so far %.3e), h err %.3e" % (s, e, worst, eh))
            assert eh <= TOL["bf16"], "step %d: h error %.3e" % (s, eh)
        assert e <= TOL["bf16"], "step %d: y error %.3e" % (s, e)
    say("  after %d steps: worst y err %.3e" % (w.steps, worst))


@pytest.mark.parametrize("shape", [(1, 1), (1, 64), (3, 100), (2, 5), (7, 1000)], ids=str)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_shapes(shape, dtype):
    nb, nd = shape
    m = ss()
    for has_D, has_z in ((False, False), (True, True), (True, False)):
        say("step %s %s D=%s z=%s" % (shape, dtype, has_D, has_z))
        inp = wl.scan_inputs(nb, 1, nd, 16, wl.F32 if dtype == "f32" else wl.BF16, has_D=has_D,
                             has_z=has_z, has_h0=True, seed=nb * 1000 + nd)
        t = {k: dev(v) for k, v in inp.items()}
        h = t["h0"].clone()
        y = m.step(h, t["u"][:, 0], t["delta"][:, 0], t["A"], t["B"][:, 0], t["C"][:, 0], D=t.get("D"),
                   z=None if t.get("z") is None else t["z"][:, 0])
        href = inp["h0"].astype(np.float64).copy()
        yref = oracle.step(href, inp["u"][:, 0], inp["delta"][:, 0], inp["A"], inp["B"][:, 0], inp["C"][:, 0],
                           D=inp["D"], z=None if inp["z"] is None else inp["z"][:, 0])
        tol = TOL[dtype]
        assert rel_err(host64(y), yref) <= tol
        assert rel_err(host64(h), href) <= tol


def test_steps_equal_scan():
    """L single steps from h0 reproduce ss_scan_fwd over the same L tokens."""
    m = ss()
    nb, nl, nd = 2, 64, 96
    inp = wl.scan_inputs(nb, nl, nd, 16, wl.F32, has_h0=True, seed=21)
    t = {k: dev(v) for k, v in inp.items()}
    say("steps vs scan")
    y_scan, h_scan = m.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"], h0=t["h0"],
                                return_last_state=True)
    h = t["h0"].clone()
    ys = []
    for s in range(nl):
        ys.append(m.step(h, t["u"][:, s].contiguous(), t["delta"][:, s].contiguous(), t["A"],
                         t["B"][:, s].contiguous(), t["C"][:, s].contiguous(), D=t["D"],
                         z=t["z"][:, s].contiguous()))
    torch.cuda.synchronize()
    y_steps = torch.stack(ys, dim=1)
    assert rel_err(host64(y_steps), host64(y_scan)) <= TOL["f32"]
    assert rel_err(host64(h), host64(h_scan)) <= TOL["f32"]


def test_step_zero_input_decays_state():
    m = ss()
    inp = wl.scan_inputs(2, 1, 64, 16, wl.BF16, has_D=True, has_z=True, has_h0=True, seed=22)
    inp["u"] = np.zeros_like(inp["u"])
    t = {k: dev(v) for k, v in inp.items()}
    h = t["h0"].clone()
    say("step zero input")
    y = m.step(h, t["u"][:, 0], t["delta"][:, 0], t["A"], t["B"][:, 0], t["C"][:, 0], D=t["D"], z=t["z"][:, 0])
    href = inp["h0"].astype(np.float64).copy()
    oracle.step(href, inp["u"][:, 0], inp["delta"][:, 0], inp["A"], inp["B"][:, 0], inp["C"][:, 0],
                D=inp["D"], z=inp["z"][:, 0])
    assert rel_err(host64(h), href) <= TOL["bf16"]
    assert np.all(np.isfinite(host64(y)))
