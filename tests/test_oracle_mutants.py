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
    ("input term drops x", "h[n] = a_bar * h[n] + b_bar * x;", "h[n] = a_bar * h[n] + b_bar;"),
    ("sign of the exponent", "exp(delta * (double)j->A[d * N + n])", "exp(-delta * (double)j->A[d * N + n])"),
    ("A transposed", "(double)j->A[d * N + n]", "(double)j->A[n * D + d]"),
    ("C read from B", "widen(j->C, srow + n, j->dtype)", "widen(j->B, srow + n, j->dtype)"),
    ("B one step late", "const double b_bar = delta * widen(j->B, srow + n, j->dtype);",
     "const double b_bar = delta * widen(j->B, (t > 0 ? srow - N : srow) + n, j->dtype);"),
    ("Bbar without delta", "const double b_bar = delta * widen(j->B, srow + n, j->dtype);",
     "const double b_bar = widen(j->B, srow + n, j->dtype);"),
    ("D skip without x", "y += (double)j->Dskip[d] * x;", "y += (double)j->Dskip[d];"),
    ("sigmoid gate instead of silu", "static double silu(double z) { return z / (1.0 + exp(-z)); }",
     "static double silu(double z) { return 1.0 / (1.0 + exp(-z)); }"),
    ("h0 ignored", "h[n] = j->h0 ? j->h0[bd * N + n] : 0.0;", "h[n] = 0.0;"),
    ("lane index swapped", "const int64_t b = bd / D, d = bd % D;",
     "const int64_t b = bd % j->batch, d = bd / j->batch;"),
    ("y from the pre-update state",
     "            h[n] = a_bar * h[n] + b_bar * x;\n        }\n        double y = 0.0;\n"
     "        for (int64_t n = 0; n < N; ++n) y += h[n] * widen(j->C, srow + n, j->dtype);",
     "            (void)0;\n        }\n        double y = 0.0;\n"
     "        for (int64_t n = 0; n < N; ++n) y += h[n] * widen(j->C, srow + n, j->dtype);\n"
     "        for (int64_t n = 0; n < N; ++n) h[n] = exp(delta * (double)j->A[d * N + n]) * h[n]"
     " + delta * widen(j->B, srow + n, j->dtype) * x;"),
    ("step forgets the decay", "hl[n] = a_bar * hl[n] + b_bar * x;", "hl[n] = hl[n] + b_bar * x;"),
    ("state recorded one step late", "j->rec_t[next_rec] == t)", "j->rec_t[next_rec] == t - 1)"),
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
