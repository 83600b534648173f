"""GPU parity of ss_ssd_fwd (the multi-head recurrence on the matrix cores) against
the fp64 oracle.  bf16 operands: max relative error (gpu_util.rel_err) <= 2e-2."""
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


def gpu_ssd(inp, return_last_state=True):
    t = {k: dev(v) for k, v in inp.items()}
    r = ss().ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t.get("D"), h0=t.get("h0"),
                     return_last_state=return_last_state)
    torch.cuda.synchronize()
    return (host64(r[0]), host64(r[1])) if return_last_state else host64(r)


CASES = [
    # (batch, seqlen, heads, dstate, has_D, has_h0)
    (1, 64, 2, 64, True, False),
    (2, 100, 3, 128, True, True),     # ragged last chunk
    (1, 1, 1, 64, False, True),       # one step
    (2, 257, 4, 128, False, False),   # several chunks, 1-row tail
    (3, 130, 2, 64, True, True),
    # dstate 256: one launch per half of the state entries, the second adding the
    # first's fp32 part of y to its own
    (2, 100, 3, 256, True, True),     # ragged last chunk
    (1, 1, 1, 256, False, True),      # one step
    (2, 257, 2, 256, False, False),   # several chunks, 1-row tail
]


@pytest.mark.parametrize("case", CASES, ids=["B%dL%dH%dN%d%s%s" % (c[:4] + ("-D" * c[4], "-h0" * c[5])) for c in CASES])
def test_ssd_small(case):
    b, l, h, n, has_D, has_h0 = case
    inp = wl.ssd_inputs(b, l, h, 64, n, has_D=has_D, has_h0=has_h0, seed=70 + l)
    say("ssd B%d L%d H%d N%d" % (b, l, h, n))
    y, hl = gpu_ssd(inp)
    ref = oracle.ssd(**inp)
    ey, eh = rel_err(y, ref["y"]), rel_err(hl, ref["h_last"])
    say("  y err %.3e, h_last err %.3e" % (ey, eh))
    assert np.all(np.isfinite(y)) and ey <= TOL["bf16"] and eh <= TOL["bf16"]


def test_ssd_degenerate_steps():
    """Step sizes the kernel treats through limits: dt = 0 rows inside chunks (no decay, no
    input: log2 dt = -inf drops the row from M and from the state update), dt = 40 rows
    (exp(dt A) underflows: the state restarts from that row), and a head with A = -1e-4
    that barely decays over the 300 rows."""
    inp = wl.ssd_inputs(2, 300, 3, 64, 128, has_D=True, has_h0=True, seed=77)
    dt = inp["dt"].copy()
    zero, big = wl.f32_to_bf16_bits(np.float32([0.0, 40.0]))
    dt[:, 5:9, :] = zero        # four rows inside the first chunk
    dt[:, 64, :] = zero         # the first row of the second chunk
    dt[:, 150, :] = big         # a reset in the middle of the third chunk
    dt[1, 255:, 0] = zero       # the tail of one head
    inp["dt"] = dt
    inp["A"] = inp["A"].copy()
    inp["A"][2] = -1e-4
    say("ssd degenerate steps")
    y, hl = gpu_ssd(inp)
    ref = oracle.ssd(**inp)
    ey, eh = rel_err(y, ref["y"]), rel_err(hl, ref["h_last"])
    say("  y err %.3e, h_last err %.3e" % (ey, eh))
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(hl))
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


def test_ssd_chaining():
    """Two calls chained through h_last -> h0 match one call over the whole sequence."""
    b, l, h, n = 2, 150, 2, 128
    inp = wl.ssd_inputs(b, l, h, 64, n, seed=80)
    say("ssd chaining")
    y_all, h_all = gpu_ssd(inp)
    cut = 70
    first = {k: (v[:, :cut] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    rest = {k: (np.ascontiguousarray(v[:, cut:]) if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    y1, h1 = gpu_ssd({k: (np.ascontiguousarray(v) if v is not None else None) for k, v in first.items()})
    rest["h0"] = h1.astype(np.float32)
    y2, h2 = gpu_ssd(rest)
    assert rel_err(np.concatenate([y1, y2], axis=1), y_all) <= TOL["bf16"]
    assert rel_err(h2, h_all) <= TOL["bf16"]


def test_ssd_layer_full():
    """The multi-head layer of the pages' example scaled to the large layer's tokens:
    B8 L2048, 64 heads of 64 channels (d_inner 4096), d_state 128; every output and every
    last-state entry of all 512 (batch row, head) pairs against the oracle (threaded)."""
    b, l, h, n = 8, 2048, 64, 128
    inp = wl.ssd_inputs(b, l, h, 64, n, seed=81)
    say("ssd layer B8 L2048 H64 N128")
    y, hl = gpu_ssd(inp)
    ref = oracle.ssd(**inp, threads=THREADS)
    ey, eh = rel_err(y, ref["y"]), rel_err(hl, ref["h_last"])
    say("  layer: y err %.3e, h_last err %.3e over all %d heads" % (ey, eh, b * h))
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]
