"""The pins must discriminate: each planted mistake in a copy of the oracle fails one.

Mistakes are planted in a temporary copy of oracle/ss_oracle.c (never in the
real file), compiled with the same flags, and the full pin suite is run on it.
"""
import os
import shutil
import subprocess

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ss_oracle.c")

# (name, exact snippet of the oracle source, replacement)
MUTANTS = [
    ("input term drops x", "return b_bar * x;", "return b_bar;"),
    ("sign of the exponent", "const double a_bar = exp(delta * a);", "const double a_bar = exp(-delta * a);"),
    ("A transposed", "            const double a = (double)j->A[d * N + n];",
     "            const double a = (double)j->A[n * D + d];"),
    ("C read from B", "y += h[n] * widen(j->C, srow + n, j->dtype)", "y += h[n] * widen(j->B, srow + n, j->dtype)"),
    ("B one step late", "input_term(delta, a, widen(j->B, srow + n, j->dtype), x, j->flags)",
     "input_term(delta, a, widen(j->B, (t > 0 ? srow - N : srow) + n, j->dtype), x, j->flags)"),
    ("Bbar without delta", "double b_bar = delta * bm; /* Euler */", "double b_bar = bm; /* Euler */"),
    ("D skip without x", "y += (double)j->Dskip[d] * x;\n        if (j->z) y *= silu(widen(j->z, row, j->dtype));",
     "y += (double)j->Dskip[d];\n        if (j->z) y *= silu(widen(j->z, row, j->dtype));"),
    ("sigmoid gate instead of silu", "static double silu(double z) { return z / (1.0 + exp(-z)); }",
     "static double silu(double z) { return 1.0 / (1.0 + exp(-z)); }"),
    ("h0 ignored", "h[n] = j->h0 ? j->h0[bd * N + n] : 0.0;", "h[n] = 0.0;"),
    ("lane index swapped", "const int64_t bd = j->lanes ? j->lanes[li] : li;\n    const int64_t b = bd / D, d = bd % D;",
     "const int64_t bd = j->lanes ? j->lanes[li] : li;\n    const int64_t b = bd % j->batch, d = bd / j->batch;"),
    ("y from the pre-update state",
     "            h[n] = a_bar * h[n] + input_term(delta, a, widen(j->B, srow + n, j->dtype), x, j->flags);\n"
     "        }\n        double y = 0.0;\n"
     "        for (int64_t n = 0; n < N; ++n) y += h[n] * widen(j->C, srow + n, j->dtype);",
     "            (void)a_bar;\n        }\n        double y = 0.0;\n"
     "        for (int64_t n = 0; n < N; ++n) y += h[n] * widen(j->C, srow + n, j->dtype);\n"
     "        for (int64_t n = 0; n < N; ++n) h[n] = exp(delta * (double)j->A[d * N + n]) * h[n]"
     " + input_term(delta, (double)j->A[d * N + n], widen(j->B, srow + n, j->dtype), x, j->flags);"),
    ("step forgets the decay", "hl[n] = a_bar * hl[n] + input_term(", "hl[n] = hl[n] + input_term("),
    ("step without its skip", "if (j->Dskip) y += (double)j->Dskip[d] * x;\n    if (j->z)", "if (j->z)"),
    ("step threads overlap", "sl[i].begin = n_lanes * i / nthreads;\n        sl[i].end = n_lanes * (i + 1) / nthreads;\n"
     "        pthread_create(&th[i], NULL, step_worker",
     "sl[i].begin = n_lanes * i / nthreads;\n        sl[i].end = n_lanes * (i + 1) / nthreads + (i + 1 < nthreads);\n"
     "        pthread_create(&th[i], NULL, step_worker"),
    ("state recorded one step late", "j->rec_t[next_rec] == t)", "j->rec_t[next_rec] == t - 1)"),
    # the delta / Bbar options
    ("ZOH ignored", "if (flags & ORACLE_ZOH) {", "if (0) {"),
    ("ZOH with the exponent's sign flipped", "expm1(da) / da;", "expm1(-da) / da;"),
    ("ZOH as a backward difference", "expm1(da) / da;", "-expm1(-da) / da;"),
    ("ZOH drops delta", "b_bar = phi * (delta * bm);", "b_bar = phi * bm;"),
    ("softplus drops its linear part", "return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v));",
     "return v > 0.0 ? log1p(exp(-v)) : log1p(exp(v));"),
    ("softplus is exp", "return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v));", "return exp(v);"),
    ("bias subtracted", "double v = raw + (delta_bias", "double v = raw - (delta_bias"),
    ("bias of channel 0 everywhere", "(double)delta_bias[d]", "(double)delta_bias[0]"),
    ("softplus always on", "return (flags & ORACLE_SOFTPLUS) ? softplus(v) : v;", "return softplus(v);"),
    # the backward
    ("adjoint not decayed", "            g[n] *= e;\n", "            (void)e;\n"),
    ("dA without the decay factor", "dA[d * N + n] += g[n] * (delta * e * hprev[n]",
     "dA[d * N + n] += g[n] * (delta * hprev[n]"),
    ("dC from the previous state", "dC[srow + n] += dyt * hcur[n];", "dC[srow + n] += dyt * hprev[n];"),
    ("dB without u", "dB[srow + n] += g[n] * beta * x;", "dB[srow + n] += g[n] * beta;"),
    ("ddelta misses the decay path", "dd += g[n] * (a * e * hprev[n] + dbeta_dd * bm * x);",
     "dd += g[n] * (dbeta_dd * bm * x);"),
    # the backward of the zero-order hold
    ("ZOH: dBbar/ddelta taken as 1", "*dbeta_ddelta = exp(x);", "*dbeta_ddelta = 1.0;"),
    ("ZOH: dBbar/dA dropped", "*dbeta_da = delta * delta * psi;", "*dbeta_da = 0.0;"),
    ("ZOH: dBbar/dA with one delta", "*dbeta_da = delta * delta * psi;", "*dbeta_da = delta * psi;"),
    ("ZOH: psi series without (k + 1)", "psi += (double)(k + 1) * xk / fact;", "psi += xk / fact;"),
    ("ZOH: psi closed form sign", "psi = (x * exp(x) - expm1(x)) / (x * x);",
     "psi = (x * exp(x) + expm1(x)) / (x * x);"),
    ("ZOH: dB with the Euler coefficient", "dB[srow + n] += g[n] * beta * x;", "dB[srow + n] += g[n] * delta * x;"),
    ("ZOH: du with the Euler coefficient", "du += g[n] * beta * bm;", "du += g[n] * delta * bm;"),
    ("silu derivative wrong", "s * (1.0 + zz * (1.0 - s))", "s * (1.0 + zz * s)"),
    ("skip uses the ungated gradient", "dD[d] += dyt * x;", "dD[d] += j->dy[row] * x;"),
    ("softplus derivative dropped", "            dd *= sigmoid(v);\n", "            (void)v;\n"),
    # the convolution
    ("conv taps reversed", "acc += (double)w[d * width + k] * widen(x, (b * seqlen + s) * x_row_stride + d, dtype);",
     "acc += (double)w[d * width + (width - 1 - k)] * widen(x, (b * seqlen + s) * x_row_stride + d, dtype);"),
    ("conv drops its oldest tap", "for (int64_t k = 0; k < width; ++k) {\n                    const int64_t s",
     "for (int64_t k = 1; k < width; ++k) {\n                    const int64_t s"),
    ("conv without its bias", "double acc = bias ? (double)bias[d] : 0.0;", "double acc = 0.0;"),
    ("conv output not through silu", "u_out[(b * seqlen + t) * dim + d] = silu(acc);",
     "u_out[(b * seqlen + t) * dim + d] = acc;"),
    ("conv rows read contiguous", "widen(x, (b * seqlen + s) * x_row_stride + d, dtype)",
     "widen(x, (b * seqlen + s) * dim + d, dtype)"),
    # the multi-head recurrence
    ("SSD decay sign flipped", "const double a = exp(d * (double)j->A[h]);", "const double a = exp(-d * (double)j->A[h]);"),
    ("SSD input without dt", "S[n * P + p] = a * S[n * P + p] + d * bn * widen(j->x, xrow + p, j->dtype);",
     "S[n * P + p] = a * S[n * P + p] + bn * widen(j->x, xrow + p, j->dtype);"),
    ("SSD output reads B", "y += S[n * P + p] * widen(j->C, srow + n, j->dtype);", "y += S[n * P + p] * widen(j->B, srow + n, j->dtype);"),
    ("SSD state transposed", "y += S[n * P + p] * widen(j->C, srow + n, j->dtype);",
     "y += S[(p % N) * P + (n % P)] * widen(j->C, srow + n, j->dtype);"),
    ("SSD dt of head 0", "const double d = widen(j->dt, (b * L + t) * H + h, j->dtype);",
     "const double d = widen(j->dt, (b * L + t) * H, j->dtype);"),
    ("dh0 before the last decay", "for (int64_t n = 0; n < N; ++n) j->dh0[bd * N + n] = g[n];",
     "for (int64_t n = 0; n < N; ++n) j->dh0[bd * N + n] = g[n] / exp(dl[0] * (double)f->A[d * N + n]);"),
]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation anchor not found once: %r" % old
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared",
                    "-o", str(lib), str(src), "-lm", "-lpthread"], check=True)
    orc = oracle.OracleLib(str(lib))
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, "no pin caught the planted mistake: %s" % name
