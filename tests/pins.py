"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` takes an oracle object exposing ``scan(...)`` and ``step(...)``
(the ``oracle`` package itself, or a deliberately broken build of it) and
raises ``AssertionError`` when the oracle disagrees.  None of them re-types the
oracle's loop: each compares with a different statement of the result.

Sources on the pages:
* Mamba walk-through (youngju.dev), section 2.2: Abar = exp(delta A), discrete
  recurrence h_t = Abar h_{t-1} + Bbar x_t, y_t = C h_t.
* same page, section 3.3: selective_scan shapes and the Euler input term
  delta*B*x; y read from the updated state.
* same page, section 3.4: D skip, y * silu(z) gate, A = -(n+1).
* LTI chapter (booiljung.github.io, 3.1), section 0.2.2: with fixed
  parameters y = x * Kbar, Kbar = (C Bbar, C Abar Bbar, ..., C Abar^{L-1} Bbar).
* LTI chapter, section 0.4.2: delta -> 0 keeps the state (Abar -> I), large
  delta with negative A resets it (Abar -> 0).
* LTI chapter, section 3.1.4.2: delta_t = Softplus(per-channel parameter +
  projection of x_t), softplus(v) = log(1 + e^v).
* Mamba walk-through, section 2.2: zero-order hold,
  Bbar = (delta A)^-1 (exp(delta A) - I) delta B; for a diagonal A it is exact
  for inputs held constant over each step, so with u = 1 and a constant B the
  state equals the continuous-time step response at every sample time.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.signal

from workloads import f32_to_bf16_bits, bf16_bits_to_f32

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f64(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _rand_case(rng, batch, seqlen, dim, dstate, *, dtype="f32", has_D=False, has_z=False,
               has_h0=False, delta_scale=0.5):
    """Small random inputs (float32, or bf16 bits) for the pins."""
    def cast(x):
        x = np.asarray(x, dtype=np.float32)
        return f32_to_bf16_bits(x) if dtype == "bf16" else x

    u = cast(rng.standard_normal((batch, seqlen, dim)))
    delta = cast(np.log1p(np.exp(rng.normal(-1.0, 0.7, (batch, seqlen, dim)))) * delta_scale * 2)
    A = (-(np.arange(1, dstate + 1))[None, :] * np.exp(rng.uniform(-0.5, 0.5, (dim, dstate)))).astype(np.float32)
    B = cast(rng.standard_normal((batch, seqlen, dstate)))
    C = cast(rng.standard_normal((batch, seqlen, dstate)))
    D = rng.standard_normal(dim).astype(np.float32) if has_D else None
    z = cast(rng.standard_normal((batch, seqlen, dim))) if has_z else None
    h0 = rng.standard_normal((batch, dim, dstate)).astype(np.float32) if has_h0 else None
    return dict(u=u, delta=delta, A=A, B=B, C=C, D=D, z=z, h0=h0)


def _close(got, want, rtol, what):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, "%s: shape %s vs %s" % (what, got.shape, want.shape)
    scale = max(float(np.max(np.abs(want))) if want.size else 0.0, 1e-300)
    err = float(np.max(np.abs(got - want))) / scale if want.size else 0.0
    assert err <= rtol, "%s: scaled error %.3e > %.1e" % (what, err, rtol)


# ---------------------------------------------------------------------------
# 1. hand-worked three-step example (tests/golden/hand_worked_3step.json)
# ---------------------------------------------------------------------------
def _eval(expr):
    return float(eval(expr, {"__builtins__": {}}, {"exp": math.exp}))


def pin_hand_worked(orc):
    with open(os.path.join(GOLDEN, "hand_worked_3step.json")) as f:
        g = json.load(f)
    L = g["shape"]["seqlen"]
    u = np.array(g["u"], dtype=np.float32).reshape(1, L, 1)
    delta = np.array(g["delta"], dtype=np.float32).reshape(1, L, 1)
    A = np.array(g["A"], dtype=np.float32)
    B = np.array(g["B"], dtype=np.float32).reshape(1, L, 2)
    C = np.array(g["C"], dtype=np.float32).reshape(1, L, 2)
    D = np.array(g["D"], dtype=np.float32)
    z = np.array(g["z"], dtype=np.float32).reshape(1, L, 1)

    plain = orc.scan(u, delta, A, B, C)
    _close(plain["y"].reshape(-1), [_eval(e) for e in g["expected_y_plain"]], 1e-14, "hand y")
    _close(plain["h_last"].reshape(-1), [_eval(e) for e in g["expected_h_last"]], 1e-14, "hand h_last")
    withd = orc.scan(u, delta, A, B, C, D=D)
    _close(withd["y"].reshape(-1), [_eval(e) for e in g["expected_y_with_D"]], 1e-14, "hand y+D")
    gated = orc.scan(u, delta, A, B, C, D=D, z=z)
    want = [_eval(a) * _eval(s) for a, s in zip(g["expected_y_with_D"], g["expected_silu_z"])]
    _close(gated["y"].reshape(-1), want, 1e-14, "hand gated y")


# ---------------------------------------------------------------------------
# 2. L = 1 closed form: h_0 = exp(delta A) h0 + delta u B, y_0 = C.h_0 (+D u)(*silu z)
# ---------------------------------------------------------------------------
def pin_single_step_closed_form(orc):
    rng = np.random.default_rng(11)
    for dtype in ("f32", "bf16"):
        for has_h0 in (False, True):
            c = _rand_case(rng, 2, 1, 5, 16, dtype=dtype, has_D=True, has_z=True, has_h0=has_h0)
            out = orc.scan(**c)
            dl = _f64(c["delta"])[:, 0, :]          # (B, D)
            x = _f64(c["u"])[:, 0, :]
            A = c["A"].astype(np.float64)
            Bm = _f64(c["B"])[:, 0, :]              # (B, N)
            Cm = _f64(c["C"])[:, 0, :]
            h = (dl * x)[:, :, None] * Bm[:, None, :]
            if has_h0:
                h = h + np.exp(dl[:, :, None] * A[None]) * c["h0"].astype(np.float64)
            y = np.einsum("bdn,bn->bd", h, Cm) + c["D"].astype(np.float64)[None] * x
            y = y * _silu(_f64(c["z"])[:, 0, :])
            _close(out["y"][:, 0, :], y, 1e-13, "L=1 y (%s, h0=%s)" % (dtype, has_h0))
            _close(out["h_last"], h, 1e-13, "L=1 h (%s, h0=%s)" % (dtype, has_h0))


# ---------------------------------------------------------------------------
# 3. LTI identity: fixed delta, B, C over time => y = causal conv(u, Kbar)
# ---------------------------------------------------------------------------
def pin_lti_convolution(orc):
    rng = np.random.default_rng(12)
    for (dim, dstate, L) in ((3, 4, 64), (5, 16, 96)):
        deltas = np.array([0.05, 0.3, 1.1, 0.7, 0.2][:dim], dtype=np.float32)
        A = (-(np.arange(1, dstate + 1))[None, :] * np.exp(rng.uniform(-0.5, 0.5, (dim, dstate)))).astype(np.float32)
        bvec = rng.standard_normal(dstate).astype(np.float32)
        cvec = rng.standard_normal(dstate).astype(np.float32)
        u = rng.standard_normal((1, L, dim)).astype(np.float32)
        delta = np.broadcast_to(deltas[None, None, :], (1, L, dim)).copy()
        B = np.broadcast_to(bvec[None, None, :], (1, L, dstate)).copy()
        C = np.broadcast_to(cvec[None, None, :], (1, L, dstate)).copy()
        y = orc.scan(u, delta, A, B, C)["y"][0]    # (L, D)

        k = np.arange(L, dtype=np.float64)
        for d in range(dim):
            dd = float(deltas[d])
            abar = np.exp(dd * A[d].astype(np.float64))                    # (N,)
            kernel = (cvec.astype(np.float64)[None, :] * abar[None, :] ** k[:, None]
                      * (dd * bvec.astype(np.float64))[None, :]).sum(axis=1)  # Kbar_k
            conv = np.convolve(u[0, :, d].astype(np.float64), kernel)[:L]
            _close(y[:, d], conv, 1e-12, "LTI convolve d=%d" % d)
            filt = np.zeros(L)
            for n in range(dstate):
                filt += cvec[n] * scipy.signal.lfilter([dd * float(bvec[n])], [1.0, -abar[n]],
                                                       u[0, :, d].astype(np.float64))
            _close(y[:, d], filt, 1e-12, "LTI lfilter d=%d" % d)


# ---------------------------------------------------------------------------
# 4. zero input: h stays exactly 0; with h0 the state only decays
# ---------------------------------------------------------------------------
def pin_zero_input(orc):
    rng = np.random.default_rng(13)
    for dtype in ("f32", "bf16"):
        c = _rand_case(rng, 2, 33, 4, 16, dtype=dtype, has_D=True, has_z=True)
        c["u"] = np.zeros_like(c["u"])
        out = orc.scan(**c)
        assert np.all(out["y"] == 0.0), "u=0, h0=0 must give y == 0 exactly"
        assert np.all(out["h_last"] == 0.0), "u=0, h0=0 must leave h == 0 exactly"
        c["h0"] = rng.standard_normal((2, 4, 16)).astype(np.float32)
        c["z"] = None
        c["D"] = None
        out = orc.scan(**c)
        total = _f64(c["delta"]).sum(axis=1)                                 # (B, D)
        want = np.exp(total[:, :, None] * c["A"].astype(np.float64)[None]) * c["h0"]
        _close(out["h_last"], want, 1e-12, "u=0 decay of h0 (%s)" % dtype)


# ---------------------------------------------------------------------------
# 5. brute force: h_t = sum_s exp(A sum_{r=s+1..t} delta_r) delta_s B_s u_s (+ decayed h0)
# ---------------------------------------------------------------------------
def brute_force(c):
    x = _f64(c["u"])
    dl = _f64(c["delta"])
    A = c["A"].astype(np.float64)
    Bm = _f64(c["B"])
    Cm = _f64(c["C"])
    nb, L, nd = x.shape
    nn = A.shape[1]
    cum = np.concatenate([np.zeros((nb, 1, nd)), np.cumsum(dl, axis=1)], axis=1)  # cum[:, t+1] = sum_{r<=t}
    y = np.zeros((nb, L, nd))
    h_last = None
    for t in range(L):
        h = np.zeros((nb, nd, nn))
        for s in range(t + 1):
            gap = cum[:, t + 1, :] - cum[:, s + 1, :]                           # sum_{r=s+1..t}
            h += np.exp(gap[:, :, None] * A[None]) * (dl[:, s, :] * x[:, s, :])[:, :, None] * Bm[:, s, None, :]
        if c.get("h0") is not None:
            h += np.exp(cum[:, t + 1, :][:, :, None] * A[None]) * c["h0"].astype(np.float64)
        y[:, t, :] = np.einsum("bdn,bn->bd", h, Cm[:, t, :])
        h_last = h
    if c.get("D") is not None:
        y += c["D"].astype(np.float64)[None, None, :] * x
    if c.get("z") is not None:
        y *= _silu(_f64(c["z"]))
    return y, h_last


def pin_brute_force(orc):
    rng = np.random.default_rng(14)
    shapes = [(1, 1, 1, 1), (2, 7, 3, 2), (1, 24, 2, 16), (3, 13, 1, 4), (2, 19, 3, 5)]
    for i, (nb, L, nd, nn) in enumerate(shapes):
        c = _rand_case(rng, nb, L, nd, nn, dtype="bf16" if i % 2 else "f32",
                       has_D=i % 2 == 0, has_z=i % 3 == 0, has_h0=i % 2 == 1)
        out = orc.scan(**c)
        y, h = brute_force(c)
        _close(out["y"], y, 1e-11, "brute force y %s" % ((nb, L, nd, nn),))
        _close(out["h_last"], h, 1e-11, "brute force h %s" % ((nb, L, nd, nn),))


# ---------------------------------------------------------------------------
# 6. geometric series: one active state, u = 1, constant delta, B = C = 1
# ---------------------------------------------------------------------------
def pin_geometric(orc):
    L, N = 50, 16
    d0 = 0.25
    A = -(np.arange(1, N + 1, dtype=np.float32))[None, :] * np.float32(1.5)
    u = np.ones((1, L, 1), dtype=np.float32)
    delta = np.full((1, L, 1), d0, dtype=np.float32)
    B = np.zeros((1, L, N), dtype=np.float32)
    C = np.zeros((1, L, N), dtype=np.float32)
    B[..., 0] = 1.0
    C[..., 0] = 1.0
    y = orc.scan(u, delta, A, B, C)["y"][0, :, 0]
    a = math.exp(d0 * float(A[0, 0]))
    t = np.arange(L)
    _close(y, d0 * (1.0 - a ** (t + 1)) / (1.0 - a), 1e-13, "geometric")


# ---------------------------------------------------------------------------
# 7. delta limits (LTI chapter, section 0.4.2)
# ---------------------------------------------------------------------------
def pin_delta_limits(orc):
    rng = np.random.default_rng(15)
    c = _rand_case(rng, 2, 9, 3, 16, has_D=True, has_h0=True)
    c["delta"] = np.zeros_like(c["delta"])
    out = orc.scan(**c)
    assert np.array_equal(out["h_last"], c["h0"].astype(np.float64)), "delta=0 must keep h bit-unchanged"
    want = np.einsum("bdn,btn->btd", c["h0"].astype(np.float64), _f64(c["C"])) \
        + c["D"].astype(np.float64)[None, None] * _f64(c["u"])
    _close(out["y"], want, 1e-14, "delta=0 output")

    c = _rand_case(rng, 1, 12, 2, 16, has_h0=True)
    c["A"] = np.broadcast_to(-(np.arange(1, 17, dtype=np.float32))[None], (2, 16)).copy()
    c["delta"] = np.full_like(c["delta"], 50.0)
    out = orc.scan(**c, record_t=[0, 5, 11])
    for k, t in enumerate([0, 5, 11]):
        want = 50.0 * _f64(c["u"])[0, t, :, None] * _f64(c["B"])[0, t, None, :]
        _close(out["h_rec"][:, k, :], want, 1e-15, "large delta resets the state, t=%d" % t)


# ---------------------------------------------------------------------------
# 8. chaining: split sequences and L single steps give the same result
# ---------------------------------------------------------------------------
def pin_chaining(orc):
    rng = np.random.default_rng(16)
    c = _rand_case(rng, 2, 40, 3, 16, dtype="bf16", has_D=True, has_z=True, has_h0=True)
    full = orc.scan(**c)
    L1 = 17
    first = orc.scan(**{k: (v[:, :L1] if k in ("u", "delta", "B", "C", "z") and v is not None else v)
                        for k, v in c.items()})
    rest = dict(c)
    for k in ("u", "delta", "B", "C", "z"):
        rest[k] = np.ascontiguousarray(c[k][:, L1:])
    rest["h0"] = first["h_last"]
    second = orc.scan(**rest)
    assert np.array_equal(np.concatenate([first["y"], second["y"]], axis=1), full["y"]), "split scan y"
    assert np.array_equal(second["h_last"], full["h_last"]), "split scan h_last"

    h = c["h0"].astype(np.float64).copy()
    for t in range(40):
        yt = orc.step(h, c["u"][:, t], c["delta"][:, t], c["A"], c["B"][:, t], c["C"][:, t],
                      D=c["D"], z=c["z"][:, t])
        assert np.array_equal(yt, full["y"][:, t]), "step y at t=%d" % t
    assert np.array_equal(h, full["h_last"]), "stepped state vs scan h_last"


# ---------------------------------------------------------------------------
# 9. causality and linearity
# ---------------------------------------------------------------------------
def pin_causality_linearity(orc):
    rng = np.random.default_rng(17)
    c = _rand_case(rng, 1, 30, 4, 16, has_D=True)
    base = orc.scan(**c)["y"]
    c2 = dict(c)
    c2["u"] = c["u"].copy()
    c2["u"][:, 10, :] += np.float32(1.0)
    pert = orc.scan(**c2)["y"]
    assert np.array_equal(pert[:, :10], base[:, :10]), "outputs before the perturbation must not change"
    assert np.all(pert[:, 10] != base[:, 10]), "the perturbed timestep must change"

    c3 = dict(c)
    c3["u"] = c["u"] * np.float32(2.0)
    assert np.array_equal(orc.scan(**c3)["y"], 2.0 * base), "y is linear in u (power-of-two scale)"
    even = c["u"].copy()
    even[:, 1::2] = 0
    odd = c["u"] - even
    ye = orc.scan(**dict(c, u=even))["y"]
    yo = orc.scan(**dict(c, u=odd))["y"]
    _close(ye + yo, base, 1e-13, "superposition")


# ---------------------------------------------------------------------------
# 10. bookkeeping: recorded states, lane subsets, threads, bf16 widening
# ---------------------------------------------------------------------------
def pin_bookkeeping(orc):
    rng = np.random.default_rng(18)
    c = _rand_case(rng, 2, 37, 5, 16, dtype="bf16", has_D=True, has_z=True, has_h0=True)
    full = orc.scan(**c, record_t=[0, 8, 36])
    for k, t in enumerate([0, 8, 36]):
        trunc = {kk: (v[:, :t + 1] if kk in ("u", "delta", "B", "C", "z") else v) for kk, v in c.items()}
        ht = orc.scan(**trunc)["h_last"].reshape(10, 16)
        assert np.array_equal(full["h_rec"][:, k], ht), "recorded state at t=%d" % t
    lanes = [7, 0, 9, 3]
    sub = orc.scan(**c, lanes=lanes)
    yfull = full["y"].transpose(0, 2, 1).reshape(10, 37)
    assert np.array_equal(sub["y"], yfull[lanes]), "lane subset y"
    assert np.array_equal(sub["h_last"], full["h_last"].reshape(10, 16)[lanes]), "lane subset h"
    thr = orc.scan(**c, threads=4)
    assert np.array_equal(thr["y"], full["y"]), "threaded run must be bit-identical"
    # the step: threads and lane subsets change nothing either
    sc = {k: (v[:, 5] if k in ("u", "delta", "B", "C", "z") else v) for k, v in c.items()}
    h1 = c["h0"].astype(np.float64).copy()
    y1 = orc.step(h1, sc["u"], sc["delta"], c["A"], sc["B"], sc["C"], D=c["D"], z=sc["z"])
    h4 = c["h0"].astype(np.float64).copy()
    y4 = orc.step(h4, sc["u"], sc["delta"], c["A"], sc["B"], sc["C"], D=c["D"], z=sc["z"], threads=4)
    assert np.array_equal(y1, y4) and np.array_equal(h1, h4), "threaded step must be bit-identical"
    hs = c["h0"].astype(np.float64).reshape(10, 16)[lanes].copy()
    ys = orc.step(hs, sc["u"], sc["delta"], c["A"], sc["B"], sc["C"], D=c["D"], z=sc["z"], lanes=lanes,
                  threads=3)
    assert np.array_equal(ys, y1.reshape(-1)[lanes]) and np.array_equal(hs, h1.reshape(10, 16)[lanes]), \
        "step lane subset"
    cf = dict(c)
    for k in ("u", "delta", "B", "C", "z"):
        cf[k] = bf16_bits_to_f32(c[k])
    assert np.array_equal(orc.scan(**cf)["y"], full["y"]), "bf16 bits widen exactly"


# ---------------------------------------------------------------------------
# 11. NumPy twin (materialised operands, recursive-doubling scan over time)
# ---------------------------------------------------------------------------
def pin_twin(orc):
    from oracle.twin import twin_scan

    rng = np.random.default_rng(19)
    for i, shp in enumerate([(1, 16, 4, 16), (2, 33, 3, 8), (3, 5, 7, 1)]):
        c = _rand_case(rng, *shp, dtype="bf16" if i == 1 else "f32", has_D=i != 2, has_z=i != 0,
                       has_h0=i == 1)
        out = orc.scan(**c)
        y, h = twin_scan(**c)
        _close(out["y"], y, 1e-13, "twin y %s" % (shp,))
        _close(out["h_last"], h, 1e-13, "twin h %s" % (shp,))
    # the options, against the twin's library routines (numpy logaddexp, scipy exprel)
    for i, (softplus, zoh) in enumerate(((True, False), (False, True), (True, True))):
        c = _rand_case(rng, 2, 21, 5, 16, dtype="bf16" if i == 2 else "f32", has_D=True, has_z=True,
                       has_h0=True)
        raw = rng.normal(-1.0, 1.5, c["u"].shape).astype(np.float32)
        c["delta"] = f32_to_bf16_bits(raw) if c["u"].dtype == np.uint16 else raw
        if not softplus:
            c["delta"] = np.abs(c["delta"]) if c["u"].dtype != np.uint16 else c["delta"] & np.uint16(0x7FFF)
        bias = rng.normal(0.0, 0.5, c["u"].shape[2]).astype(np.float32)
        opts = dict(delta_bias=bias if softplus else None, delta_softplus=softplus, zoh=zoh)
        out = orc.scan(**c, **opts)
        y, h = twin_scan(**c, **opts)
        _close(out["y"], y, 1e-12, "twin y, softplus=%s zoh=%s" % (softplus, zoh))
        _close(out["h_last"], h, 1e-12, "twin h, softplus=%s zoh=%s" % (softplus, zoh))


# ---------------------------------------------------------------------------
# 12. zero-order hold = exact continuous-time step response
#     h' = A h + B u with u = 1 and B constant: h(T) = e^{AT} h0 + (B/A)(e^{AT} - 1),
#     T = delta_0 + ... + delta_t, whatever the step sizes; A = 0 integrates: h0 + B T
# ---------------------------------------------------------------------------
def pin_zoh_step_response(orc):
    rng = np.random.default_rng(23)
    nb, nl, nd, nn = 2, 40, 3, 4
    A = -rng.uniform(0.2, 3.0, (nd, nn)).astype(np.float32)
    A[0, 0] = 0.0
    A[1, 1] = 0.3  # a growing mode obeys the same formula
    delta = rng.uniform(0.01, 0.8, (nb, nl, nd)).astype(np.float32)
    u = np.ones((nb, nl, nd), dtype=np.float32)
    beta = rng.standard_normal((nb, nn)).astype(np.float32)
    Bm = np.repeat(beta[:, None, :], nl, axis=1)
    Cm = rng.standard_normal((nb, nl, nn)).astype(np.float32)
    h0 = rng.standard_normal((nb, nd, nn)).astype(np.float32)
    out = orc.scan(u, delta, A, Bm, Cm, h0=h0, zoh=True)
    T = np.cumsum(delta.astype(np.float64), axis=1)[..., None]           # (B, L, D, 1)
    a = A.astype(np.float64)[None, None]                                  # (1, 1, D, N)
    at = a * T
    safe = np.where(a == 0.0, 1.0, a)
    growth = np.where(a == 0.0, T, np.expm1(at) / safe)                   # (e^{AT} - 1)/A, or T
    h = np.exp(at) * h0.astype(np.float64)[:, None] + beta.astype(np.float64)[:, None, None, :] * growth
    y = np.einsum("bldn,bln->bld", h, Cm.astype(np.float64))
    _close(out["y"], y, 1e-11, "ZOH step response y")
    _close(out["h_last"], h[:, -1], 1e-11, "ZOH step response h_last")


# ---------------------------------------------------------------------------
# 13. zero-order hold, one step from zero: the input term is exprel(delta A)
#     times Euler's (scipy's exprel(x) = (e^x - 1)/x); a huge step with A < 0
#     lands on the equilibrium -B u / A; A = 0 is Euler bit for bit
# ---------------------------------------------------------------------------
def pin_zoh_limits(orc):
    import scipy.special

    rng = np.random.default_rng(24)
    c = _rand_case(rng, 2, 1, 6, 16)
    zoh = orc.scan(**c, zoh=True)["h_last"]
    euler = orc.scan(**c)["h_last"]
    da = _f64(c["delta"])[:, 0, :, None] * c["A"].astype(np.float64)[None]
    _close(zoh, scipy.special.exprel(da) * euler, 1e-14, "ZOH / Euler = exprel(delta A)")

    c["delta"] = np.full_like(c["delta"], 1.0e4)
    c["h0"] = rng.standard_normal((2, 6, 16)).astype(np.float32)
    big = orc.scan(**c, zoh=True)["h_last"]
    bu = _f64(c["B"])[:, 0, None, :] * _f64(c["u"])[:, 0, :, None]
    _close(big, -bu / c["A"].astype(np.float64)[None], 1e-14, "ZOH huge step -> -B u / A")

    c = _rand_case(rng, 2, 9, 4, 8, has_h0=True)
    c["A"] = np.zeros_like(c["A"])
    a0 = orc.scan(**c, zoh=True)
    e0 = orc.scan(**c)
    assert np.array_equal(a0["y"], e0["y"]) and np.array_equal(a0["h_last"], e0["h_last"]), "A = 0: ZOH is Euler"


# ---------------------------------------------------------------------------
# 14. step size softplus(delta + bias[d]), softplus(v) = log(1 + e^v):
#     softplus(0) = ln 2 and 2^A = e^{ln2 A}; a per-channel bias; no overflow
#     at +-1000; a bias without softplus is a plain shift
# ---------------------------------------------------------------------------
def pin_softplus_bias(orc):
    rng = np.random.default_rng(25)
    c = _rand_case(rng, 2, 1, 5, 16, has_h0=True)
    h0 = c["h0"].astype(np.float64)
    bu = _f64(c["B"])[:, 0, None, :] * _f64(c["u"])[:, 0, :, None]      # (B, D, N)
    A = c["A"].astype(np.float64)[None]

    c["delta"] = np.zeros_like(c["delta"])
    got = orc.scan(**c, delta_softplus=True)["h_last"]
    _close(got, np.exp2(A) * h0 + math.log(2.0) * bu, 1e-14, "softplus(0) = ln 2")

    bias = np.array([-3.0, -0.5, 0.0, 0.75, 4.0], dtype=np.float32)
    got = orc.scan(**c, delta_softplus=True, delta_bias=bias)["h_last"]
    dl = np.logaddexp(0.0, bias.astype(np.float64))[None, :, None]         # log(1 + e^b) per channel
    _close(got, np.exp(dl * A) * h0 + dl * bu, 1e-14, "softplus(bias[d])")

    c["delta"] = np.full_like(c["delta"], 1000.0)
    got = orc.scan(**c, delta_softplus=True)["h_last"]
    _close(got, 1000.0 * bu, 1e-14, "softplus(1000) = 1000, e^{1000 A} = 0")
    c["delta"] = np.full_like(c["delta"], -1000.0)
    got = orc.scan(**c, delta_softplus=True)
    assert np.array_equal(got["h_last"], h0), "softplus(-1000) = 0 keeps the state"

    c["delta"] = np.full_like(c["delta"], 0.25)
    shift = np.full(5, 0.5, dtype=np.float32)
    got = orc.scan(**c, delta_bias=shift)["h_last"]
    _close(got, np.exp(0.75 * A) * h0 + 0.75 * bu, 1e-14, "bias without softplus")

    # the recurrent step takes the same options
    st = _rand_case(rng, 3, 1, 4, 16, has_h0=True)
    bias4 = rng.normal(0.0, 1.0, 4).astype(np.float32)
    for opts in (dict(delta_softplus=True, delta_bias=bias4), dict(zoh=True),
                 dict(delta_softplus=True, zoh=True)):
        h = st["h0"].astype(np.float64).copy()
        y = orc.step(h, st["u"][:, 0], st["delta"][:, 0], st["A"], st["B"][:, 0], st["C"][:, 0], **opts)
        ref = orc.scan(**st, **opts)
        _close(y, ref["y"][:, 0, :], 1e-15, "step == one scan step %s" % sorted(opts))
        _close(h, ref["h_last"], 1e-15, "step state %s" % sorted(opts))


# ---------------------------------------------------------------------------
# 15. backward: every gradient element against torch's fp64 autograd of a torch
#     statement of the forward (library reverse mode, no hand-derived adjoint)
# ---------------------------------------------------------------------------
def _torch_forward(c, softplus, zoh=False):
    import torch

    f64 = lambda a: None if a is None else torch.tensor(_f64(a), dtype=torch.float64, requires_grad=True)  # noqa: E731
    t = {k: f64(c.get(k)) for k in ("u", "delta", "A", "B", "C", "D", "z", "h0", "delta_bias")}
    dl = t["delta"]
    if t["delta_bias"] is not None:
        dl = dl + t["delta_bias"][None, None, :]
    if softplus:
        dl = torch.logaddexp(torch.zeros_like(dl), dl)
    nb, nl, nd = dl.shape
    if t["h0"] is None:  # a zero initial state still has a gradient
        t["h0"] = torch.zeros(nb, nd, t["A"].shape[1], dtype=torch.float64, requires_grad=True)
    h = t["h0"]
    ys = []
    for s_ in range(nl):
        da = dl[:, s_, :, None] * t["A"][None]
        bbar = dl[:, s_, :, None] * t["B"][:, s_, None, :]
        if zoh:  # (delta A)^-1 (exp(delta A) - 1) delta B; the cases keep delta A away from 0
            bbar = torch.expm1(da) / da * bbar
        h = torch.exp(da) * h + bbar * t["u"][:, s_, :, None]
        ys.append((h * t["C"][:, s_, None, :]).sum(-1))
    y = torch.stack(ys, 1)
    if t["D"] is not None:
        y = y + t["D"][None, None, :] * t["u"]
    if t["z"] is not None:
        y = y * torch.nn.functional.silu(t["z"])
    return t, y, h


def pin_bwd_autograd(orc):
    import torch

    rng = np.random.default_rng(26)
    cases = [((2, 11, 5, 8), dict(dtype="f32", has_D=True, has_z=True, has_h0=True), False, True, False),
             ((1, 17, 3, 16), dict(dtype="bf16", has_D=True, has_z=False, has_h0=False), True, False, False),
             ((3, 6, 4, 4), dict(dtype="f32", has_D=False, has_z=True, has_h0=True), True, True, False),
             # zero-order hold: step sizes from 1e-5 to 3, so that delta*A falls on both sides of
             # the oracle's switch from the series of psi to its closed form
             ((2, 13, 4, 8), dict(dtype="f32", has_D=True, has_z=True, has_h0=True), False, True, True),
             ((1, 9, 3, 4), dict(dtype="f32", has_D=False, has_z=False, has_h0=True), True, False, True)]
    for shp, kw, softplus, with_dh, zoh in cases:
        c = _rand_case(rng, *shp, **kw)
        if zoh and not softplus:
            c["delta"] = np.exp(rng.uniform(np.log(1e-5), np.log(3.0), c["u"].shape)).astype(np.float32)
        if softplus:
            raw = rng.normal(-1.0, 1.0, c["u"].shape).astype(np.float32)
            c["delta"] = f32_to_bf16_bits(raw) if c["u"].dtype == np.uint16 else raw
            c["delta_bias"] = rng.normal(0.0, 0.7, shp[2]).astype(np.float32)
        dy = rng.standard_normal(shp[:3])
        dhl = rng.standard_normal((shp[0], shp[2], shp[3])) if with_dh else None
        got = orc.scan_bwd(**c, dy=dy, dh_last=dhl, delta_softplus=softplus, zoh=zoh)
        t, y, h = _torch_forward(c, softplus, zoh)
        loss = (y * torch.tensor(dy)).sum()
        if with_dh:
            loss = loss + (h * torch.tensor(dhl)).sum()
        loss.backward()
        names = {"du": "u", "ddelta": "delta", "dA": "A", "dB": "B", "dC": "C", "dD": "D", "dz": "z",
                 "dh0": "h0", "ddelta_bias": "delta_bias"}
        for gk, ik in names.items():
            if t[ik] is None:
                assert gk not in got, "%s present without %s" % (gk, ik)
                continue
            _close(got[gk], t[ik].grad.numpy(), 1e-11, "autograd %s %s zoh=%s" % (gk, shp, zoh))


# ---------------------------------------------------------------------------
# 16. backward: directional derivatives against fp64 central differences of
#     the NumPy twin's forward (one random direction per input), Euler and
#     zero-order hold
# ---------------------------------------------------------------------------
def pin_bwd_finite_differences(orc):
    from oracle.twin import twin_scan

    rng = np.random.default_rng(27)
    for zoh in (False, True):
        c = _rand_case(rng, 2, 9, 3, 4, dtype="f32", has_D=True, has_z=True, has_h0=True)
        raw = rng.normal(-0.5, 1.0, c["u"].shape).astype(np.float32)
        if zoh:  # some step sizes near 0 (the series side of psi) and a channel with A = 0
            raw[:, ::3, :] = -12.0
            c["A"][1, :] = 0.0
        c["delta"] = raw
        c["delta_bias"] = rng.normal(0.0, 0.5, 3).astype(np.float32)
        dy = rng.standard_normal((2, 9, 3))
        dhl = rng.standard_normal((2, 3, 4))
        grads = orc.scan_bwd(**c, dy=dy, dh_last=dhl, delta_softplus=True, zoh=zoh)

        base = {k: (None if v is None else _f64(v)) for k, v in c.items()}

        def loss(inp):
            y, h = twin_scan(**inp, delta_softplus=True, zoh=zoh)
            return float(np.sum(y * dy) + np.sum(h * dhl))

        eps = 1e-6
        for gk, ik in (("du", "u"), ("ddelta", "delta"), ("dA", "A"), ("dB", "B"), ("dC", "C"), ("dD", "D"),
                       ("dz", "z"), ("dh0", "h0"), ("ddelta_bias", "delta_bias")):
            v = rng.standard_normal(base[ik].shape)
            plus = dict(base)
            minus = dict(base)
            plus[ik] = base[ik] + eps * v
            minus[ik] = base[ik] - eps * v
            fd = (loss(plus) - loss(minus)) / (2 * eps)
            an = float(np.sum(grads[gk] * v))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), \
                "finite differences %s zoh=%s: %.9g vs %.9g" % (gk, zoh, an, fd)
        if zoh:  # the A = 0 channel's dA alone, where the closed form of dBbar/dA is 0/0
            v = np.zeros_like(base["A"])
            v[1, :] = rng.standard_normal(4)
            plus, minus = dict(base), dict(base)
            plus["A"], minus["A"] = base["A"] + eps * v, base["A"] - eps * v
            fd = (loss(plus) - loss(minus)) / (2 * eps)
            an = float(np.sum(grads["dA"] * v))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), "finite differences dA at A = 0: %.9g vs %.9g" % (an, fd)


# ---------------------------------------------------------------------------
# 17. causal depthwise convolution + SiLU (walk-through section 3.4): against
#     torch's fp64 grouped conv1d with the block's padding and truncation; the
#     impulse response; causality; the x half of a (B, L, 2D) projection read
#     in place
# ---------------------------------------------------------------------------
def pin_conv1d_silu(orc):
    import torch

    rng = np.random.default_rng(28)
    for (nb, nl, nd, width, dtype) in ((2, 40, 7, 4, "f32"), (1, 33, 16, 3, "bf16"), (3, 5, 4, 6, "f32")):
        x = rng.standard_normal((nb, nl, nd)).astype(np.float32)
        if dtype == "bf16":
            x = f32_to_bf16_bits(x)
        wt = rng.standard_normal((nd, width)).astype(np.float32)
        bias = rng.standard_normal(nd).astype(np.float32)
        got = orc.conv1d_silu(x, wt, bias)
        xt = torch.tensor(_f64(x)).transpose(1, 2)                       # (B, D, L)
        ref = torch.nn.functional.conv1d(xt, torch.tensor(wt, dtype=torch.float64)[:, None, :],
                                         torch.tensor(bias, dtype=torch.float64), padding=width - 1,
                                         groups=nd)[:, :, :nl]
        ref = torch.nn.functional.silu(ref).transpose(1, 2).numpy()
        _close(got, ref, 1e-13, "conv1d vs torch (%d,%d,%d,w%d)" % (nb, nl, nd, width))
        # no bias = bias of zeros
        _close(orc.conv1d_silu(x, wt), orc.conv1d_silu(x, wt, np.zeros(nd, np.float32)), 0.0, "no bias")

    # impulse at t0 in channel 1: silu(bias + w[1, width-1-(t-t0)]) for t0 <= t < t0+width, silu(bias) elsewhere
    nl, nd, width, t0 = 20, 3, 4, 6
    x = np.zeros((1, nl, nd), np.float32)
    x[0, t0, 1] = 1.0
    wt = rng.standard_normal((nd, width)).astype(np.float32)
    bias = rng.standard_normal(nd).astype(np.float32)
    got = orc.conv1d_silu(x, wt, bias)[0, :, 1]
    pre = np.full(nl, float(bias[1]))
    for t in range(t0, t0 + width):
        pre[t] += float(wt[1, width - 1 - (t - t0)])
    _close(got, _silu(pre), 1e-15, "conv1d impulse response")

    # causality: changing x at t1 leaves u before t1 bit-identical
    x = rng.standard_normal((2, 30, 5)).astype(np.float32)
    wt = rng.standard_normal((5, 4)).astype(np.float32)
    a = orc.conv1d_silu(x, wt)
    x2 = x.copy()
    x2[:, 17:, :] += 1.0
    b = orc.conv1d_silu(x2, wt)
    assert np.array_equal(a[:, :17], b[:, :17]) and not np.array_equal(a[:, 17:], b[:, 17:]), "conv1d causality"

    # the x half of xz (B, L, 2D) read in place equals the contiguous copy
    xz = f32_to_bf16_bits(rng.standard_normal((2, 12, 10)).astype(np.float32))
    wt = rng.standard_normal((5, 4)).astype(np.float32)
    assert np.array_equal(orc.conv1d_silu(xz, wt, dim=5), orc.conv1d_silu(np.ascontiguousarray(xz[:, :, :5]), wt)), \
        "conv1d strided rows"


# ---------------------------------------------------------------------------
# 18. multi-head recurrence (walk-through section 4.1): its dual, the causal
#     structured matrix applied to the inputs,
#       y_t = sum_{s<=t} (C_t . B_s) exp(A sum_{s<r<=t} dt_r) dt_s x_s + exp(A sum_{r<=t} dt_r) C_t . h0 + D x_t,
#     materialised as an L x L matrix per head; and its reduction to the
#     selective scan (every head channel is a scan channel with A broadcast over
#     the state entries and the head's dt); chaining
# ---------------------------------------------------------------------------
def _ssd_case(rng, nb, nl, nh, hp, ns, dtype="f32", has_D=True, has_h0=True):
    def cast(a):
        a = np.asarray(a, dtype=np.float32)
        return f32_to_bf16_bits(a) if dtype == "bf16" else a

    x = cast(rng.standard_normal((nb, nl, nh, hp)))
    dt = cast(np.log1p(np.exp(rng.normal(-1.5, 0.8, (nb, nl, nh)))))
    A = -np.exp(rng.uniform(-1.0, 1.0, nh)).astype(np.float32)
    B = cast(rng.standard_normal((nb, nl, ns)))
    C = cast(rng.standard_normal((nb, nl, ns)))
    D = rng.standard_normal(nh).astype(np.float32) if has_D else None
    h0 = rng.standard_normal((nb, nh, ns, hp)).astype(np.float32) if has_h0 else None
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, h0=h0)


def pin_ssd_dual_form(orc):
    rng = np.random.default_rng(29)
    for (nb, nl, nh, hp, ns, dtype) in ((2, 13, 3, 4, 5, "f32"), (1, 21, 2, 8, 16, "bf16")):
        c = _ssd_case(rng, nb, nl, nh, hp, ns, dtype)
        got = orc.ssd(**c)
        x, dt, B, C = _f64(c["x"]), _f64(c["dt"]), _f64(c["B"]), _f64(c["C"])
        A = c["A"].astype(np.float64)
        y = np.zeros((nb, nl, nh, hp))
        for b in range(nb):
            for h in range(nh):
                cum = np.cumsum(dt[b, :, h])                      # sum_{r<=t} dt_r
                seg = cum[:, None] - cum[None, :]                 # sum_{s<r<=t} dt_r
                Lmat = np.where(np.tril(np.ones((nl, nl))) > 0, np.exp(A[h] * seg), 0.0)
                M = Lmat * (C[b] @ B[b].T)                        # (T o M) of the dual form
                y[b, :, h] = M @ (dt[b, :, h, None] * x[b, :, h])
                y[b, :, h] += np.exp(A[h] * cum)[:, None] * (C[b] @ c["h0"][b, h].astype(np.float64))
                y[b, :, h] += c["D"][h] * x[b, :, h]
        _close(got["y"], y, 1e-12, "SSD dual form (%d,%d,%d,%d,%d)" % (nb, nl, nh, hp, ns))


def pin_ssd_reduces_to_scan(orc):
    rng = np.random.default_rng(30)
    nb, nl, nh, hp, ns = 2, 17, 3, 4, 16
    c = _ssd_case(rng, nb, nl, nh, hp, ns)
    got = orc.ssd(**c)
    d = nh * hp
    u = c["x"].reshape(nb, nl, d)
    delta = np.repeat(c["dt"], hp, axis=2)                            # channel h*P + p takes dt of head h
    A = np.repeat(c["A"], hp)[:, None] * np.ones((1, ns), np.float32)
    Dskip = np.repeat(c["D"], hp)
    h0 = c["h0"].transpose(0, 1, 3, 2).reshape(nb, d, ns)             # (B, H, N, P) -> (B, H*P, N)
    ref = orc.scan(u, delta, A.astype(np.float32), c["B"], c["C"], D=Dskip, h0=h0)
    _close(got["y"].reshape(nb, nl, d), ref["y"], 1e-13, "SSD as a selective scan")
    _close(got["h_last"].transpose(0, 1, 3, 2).reshape(nb, d, ns), ref["h_last"], 1e-13, "SSD state as scan state")
    # chaining: the first 9 steps then the rest from their state
    first = {k: (v[:, :9] if k in ("x", "dt", "B", "C") else v) for k, v in c.items()}
    rest = {k: (v[:, 9:] if k in ("x", "dt", "B", "C") else v) for k, v in c.items()}
    a = orc.ssd(**first)
    rest["h0"] = a["h_last"]
    b = orc.ssd(**rest)
    assert np.array_equal(np.concatenate([a["y"], b["y"]], axis=1), got["y"]), "SSD chaining"
    sel = [1, 4, 5]
    part = orc.ssd(**c, heads=sel)
    assert np.array_equal(part["y"], got["y"].transpose(0, 2, 1, 3).reshape(nb * nh, nl, hp)[sel]), "SSD head subset"
    thr = orc.ssd(**c, threads=4)
    assert np.array_equal(thr["y"], got["y"]) and np.array_equal(thr["h_last"], got["h_last"]), \
        "threaded SSD must be bit-identical"
    part3 = orc.ssd(**c, heads=sel, threads=2)
    assert np.array_equal(part3["y"], part["y"]), "threaded SSD head subset"


ALL_PINS = [pin_hand_worked, pin_single_step_closed_form, pin_lti_convolution, pin_zero_input,
            pin_brute_force, pin_geometric, pin_delta_limits, pin_chaining,
            pin_causality_linearity, pin_bookkeeping, pin_twin, pin_zoh_step_response,
            pin_zoh_limits, pin_softplus_bias, pin_bwd_autograd, pin_bwd_finite_differences, pin_conv1d_silu,
            pin_ssd_dual_form, pin_ssd_reduces_to_scan]
