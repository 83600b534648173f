"""The scan, its backward and the multi-head recurrence at the largest slab the kernels
address.

Rows of the (B, L, D) streams are reached through 32-bit buffer offsets, so the
library rejects a chunk (forward) or a batch row (backward) of 2 GiB or more.
These tests run fp32 shapes just under that limit: one batch row of L = 65543
rows of D = 8191 channels is 2 147 450 852 bytes, 32 796 below 2^31, and the
last 64-channel block has an idle lane whose offsets sit above the range (the
largest, 2^31 plus the last row's offset, stays below 2^32).  The
inputs are drawn on the device (torch's seeded generator, the workloads'
distributions); the oracle checks a sample of channels over the whole sequence,
which is exact because channels are independent.  For the backward, dy and
dh_last are zero outside the sampled channels: every other channel then
contributes exact zeros, so the channel sums dB and dC are the oracle's sums
over the sampled channels, and the other channels' gradients must be exactly 0.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import TOL, dev, host64, rel_err, say

pytestmark = pytest.mark.gpu

NB, NL, ND, NS = 1, 65543, 8191, 16
SEL = np.array([0, 1, 63, 64, 2047, 4095, 4096, 6000, 8127, 8128, 8189, 8190], dtype=np.int64)


def ss():
    import selective_state_space_85_amd as m

    return m


def device_inputs(seed):
    """fp32 inputs on the device: u, z ~ N(0, 1); delta = softplus(N(-2, 1)); B, C ~ N(0, 1);
    A = -(n+1) exp(U(-1/2, 1/2)); D ~ N(0, 1); h0 ~ N(0, 1)."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    shp = (NB, NL, ND)
    t = {"u": torch.randn(shp, device="cuda", generator=g),
         "delta": torch.nn.functional.softplus(torch.randn(shp, device="cuda", generator=g) - 2.0),
         "z": torch.randn(shp, device="cuda", generator=g),
         "B": torch.randn(NB, NL, NS, device="cuda", generator=g),
         "C": torch.randn(NB, NL, NS, device="cuda", generator=g),
         "A": torch.from_numpy(wl.make_A(ND, NS, True, seed=seed)).cuda(),
         "D": torch.randn(ND, device="cuda", generator=g),
         "h0": torch.randn(NB, ND, NS, device="cuda", generator=g)}
    assert 0 < 2 ** 31 - NL * ND * 4 < 2 ** 16  # within 64 KB of the limit
    assert 2 ** 31 + (NL - 1) * ND * 4 < 2 ** 32
    return t


def sampled(t):
    """The oracle's sub-problem: the sampled channels, as float32 host arrays."""
    sel = torch.from_numpy(SEL).cuda()
    cols = lambda x: np.ascontiguousarray(x.index_select(2, sel).cpu().numpy())  # noqa: E731
    return dict(u=cols(t["u"]), delta=cols(t["delta"]), z=cols(t["z"]), B=t["B"].cpu().numpy(),
                C=t["C"].cpu().numpy(), A=t["A"].cpu().numpy()[SEL], D=t["D"].cpu().numpy()[SEL],
                h0=np.ascontiguousarray(t["h0"].cpu().numpy()[:, SEL]))


def test_forward_at_the_chunk_slab_limit():
    m = ss()
    t = device_inputs(1201)
    say("forward, one chunk of %d x %d fp32 (%d bytes)" % (NL, ND, NL * ND * 4))
    y, hl = m.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"], h0=t["h0"], chunk_len=NL,
                       return_last_state=True)
    torch.cuda.synchronize()
    assert m.scan_plan(NB, NL, ND, NS, NL) == (NL, 1)
    ref = oracle.scan(**sampled(t))
    ey = rel_err(host64(y[:, :, torch.from_numpy(SEL).cuda()]), ref["y"])
    eh = rel_err(host64(hl[:, torch.from_numpy(SEL).cuda()]), ref["h_last"])
    say("  y err %.2e, h_last err %.2e" % (ey, eh))
    assert ey <= TOL["f32"] and eh <= TOL["f32"]
    assert torch.isfinite(y).all().item()


def test_backward_at_the_row_slab_limit():
    m = ss()
    t = device_inputs(1202)
    sel = torch.from_numpy(SEL).cuda()
    g = torch.Generator(device="cuda").manual_seed(1203)
    dy = torch.zeros(NB, NL, ND, device="cuda")
    dy[:, :, sel] = torch.randn(NB, NL, SEL.size, device="cuda", generator=g)
    dhl = torch.zeros(NB, ND, NS, device="cuda")
    dhl[:, sel] = torch.randn(NB, SEL.size, NS, device="cuda", generator=g)
    say("backward, one batch row of %d x %d fp32 (%d bytes)" % (NL, ND, NL * ND * 4))
    gr = m.scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dy, D=t["D"], z=t["z"], h0=t["h0"], dh_last=dhl)
    torch.cuda.synchronize()
    sub = sampled(t)
    ref = oracle.scan_bwd(**sub, dy=np.ascontiguousarray(dy.index_select(2, sel).cpu().numpy()),
                          dh_last=np.ascontiguousarray(dhl[:, sel].cpu().numpy()))
    errs = {}
    for k in ("du", "ddelta", "dz"):
        errs[k] = rel_err(host64(gr[k].index_select(2, sel)), ref[k])
        rest = gr[k].clone()
        rest[:, :, sel] = 0
        assert torch.count_nonzero(rest).item() == 0, "%s of a channel without gradient" % k
    for k in ("dA", "dD"):
        errs[k] = rel_err(host64(gr[k][sel]), ref[k])
        rest = gr[k].clone()
        rest[sel] = 0
        assert torch.count_nonzero(rest).item() == 0, "%s of a channel without gradient" % k
    errs["dh0"] = rel_err(host64(gr["dh0"][:, sel]), ref["dh0"])
    for k in ("dB", "dC"):
        errs[k] = rel_err(host64(gr[k]), ref[k])
    say("  " + ", ".join("%s %.1e" % kv for kv in errs.items()))
    for k, e in errs.items():
        assert e <= TOL["f32"], "%s error %.3e" % (k, e)


def bf16_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("nn", [64, 256])
def test_ssd_at_the_row_slab_limit(nn):
    """The multi-head recurrence with one batch row of x just under 2 GiB: 256 heads of 64
    channels, bf16, L the longest the library accepts at this width: 65535 at dstate 64;
    65472 at dstate 256, where the fp32 part of y (twice the bytes of y, with the rows a
    ragged last chunk reaches) must stay below 2^32.  The oracle checks the first and the
    last head over the whole sequence."""
    nh = 256
    nl = 65535 if nn == 64 else 65472
    if nn == 64:
        assert 0 < 2 ** 31 - nl * nh * 64 * 2 < 2 ** 16   # x within 64 KB of 2 GiB
    else:
        assert 2 * (nl + 63) * nh * 128 < 2 ** 32 <= 2 * (nl + 64 + 63) * nh * 128
    g = torch.Generator(device="cuda").manual_seed(1204)
    x = torch.randn(1, nl, nh, 64, device="cuda", generator=g).to(torch.bfloat16)
    dt = torch.nn.functional.softplus(torch.randn(1, nl, nh, device="cuda", generator=g) - 2.0).to(torch.bfloat16)
    A = -(torch.rand(nh, device="cuda", generator=g) * 15.0 + 1.0)
    B = torch.randn(1, nl, nn, device="cuda", generator=g).to(torch.bfloat16)
    C = torch.randn(1, nl, nn, device="cuda", generator=g).to(torch.bfloat16)
    D = torch.randn(nh, device="cuda", generator=g)
    h0 = torch.randn(1, nh, nn, 64, device="cuda", generator=g)
    say("ssd, one batch row of %d x %d heads x 64 bf16 (%d bytes)" % (nl, nh, nl * nh * 128))
    y, hl = ss().ssd_fwd(x, dt, A, B, C, D=D, h0=h0, return_last_state=True)
    torch.cuda.synchronize()
    heads = [0, nh - 1]
    sel = torch.tensor(heads, device="cuda")
    ref = oracle.ssd(bf16_bits(x.index_select(2, sel)), bf16_bits(dt.index_select(2, sel)), A[sel].cpu().numpy(),
                     bf16_bits(B), bf16_bits(C), D=D[sel].cpu().numpy(), h0=h0[:, sel].cpu().numpy())
    ey = rel_err(host64(y.index_select(2, sel)), ref["y"])
    eh = rel_err(host64(hl[:, sel]), ref["h_last"])
    say("  y err %.2e, h_last err %.2e" % (ey, eh))
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


def test_step_rows_over_one_launch():
    """ss_step over more batch rows than one launch's grid covers (65535 grid rows of two
    batch rows each): 131075 rows of 24 channels, bf16, skip, gate and h0, in two launches.
    Every output and state against the oracle."""
    nb, nd = 2 * 65535 + 5, 24
    m = ss()
    inp = wl.scan_inputs(nb, 1, nd, NS, wl.BF16, has_D=True, has_z=True, has_h0=True, seed=31)
    t = {k: dev(v) for k, v in inp.items()}
    h = t["h0"].clone()
    say("step over two launches: B=%d D=%d" % (nb, nd))
    y = m.step(h, t["u"][:, 0].contiguous(), t["delta"][:, 0].contiguous(), t["A"], t["B"][:, 0].contiguous(),
               t["C"][:, 0].contiguous(), D=t["D"], z=t["z"][:, 0].contiguous())
    href = inp["h0"].astype(np.float64).copy()
    yref = oracle.step(href, np.ascontiguousarray(inp["u"][:, 0]), np.ascontiguousarray(inp["delta"][:, 0]),
                       inp["A"], np.ascontiguousarray(inp["B"][:, 0]), np.ascontiguousarray(inp["C"][:, 0]),
                       D=inp["D"], z=np.ascontiguousarray(inp["z"][:, 0]), threads=16)
    ey, eh = rel_err(host64(y), yref), rel_err(host64(h), href)
    say("  y err %.3e, h err %.3e" % (ey, eh))
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


def test_panel_over_one_launch():
    """The B/C panel pass over more (batch row, chunk) pairs than one launch's grid covers:
    33000 batch rows of 40 rows in chunks of 16 (3 chunks, the last ragged), with the
    checkpointing forward, whose chunked plans keep the panel.  Every output against the
    oracle."""
    nb, nl, nd = 33000, 40, 8
    m = ss()
    inp = wl.scan_inputs(nb, nl, nd, NS, wl.BF16, has_D=True, has_z=True, has_h0=True, seed=32)
    t = {k: dev(v) for k, v in inp.items()}
    T, K = m.scan_plan(nb, nl, nd, NS, chunk_len=16)
    assert (T, K) == (16, 3) and nb * K > 65535
    ck = torch.empty(m.scan_ckpt_shape(nb, nl, nd, NS), device="cuda")
    say("panel over two launches: B=%d L=%d D=%d, %d chunks" % (nb, nl, nd, K))
    y, hl = m.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"], h0=t["h0"],
                       return_last_state=True, chunk_len=16, ckpt=ck)
    ref = oracle.scan(**inp, threads=16)
    ey, eh = rel_err(host64(y), ref["y"]), rel_err(host64(hl), ref["h_last"])
    say("  y err %.3e, h_last err %.3e" % (ey, eh))
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]
