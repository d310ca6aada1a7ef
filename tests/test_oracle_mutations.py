"""The pins are strong enough: each plausible mistake planted in a copy of the
oracle (a dropped term, a wrong sign, a wrong index or operand) must make at
least one pin fail.  Mistakes are planted only in temporary copies of the C
source, built with gcc on the CPU; the real oracle is never touched."""
import os
import subprocess

import pytest

import oracle_pins as P
from oracle import oracle as O

SRC = os.path.join(os.path.dirname(O.__file__), "gdn_oracle.c")

# (name, exact text in gdn_oracle.c, replacement)
MUTANTS = [
    ("no decay on carried state",
     "Si[j] = a * Si[j] - a * b * w * k[j]", "Si[j] = Si[j] - a * b * w * k[j]"),
    ("no decay on erase term",
     "Si[j] = a * Si[j] - a * b * w * k[j]", "Si[j] = a * Si[j] - b * w * k[j]"),
    ("no write strength on write term",
     "+ b * v[i] * k[j];", "+ v[i] * k[j];"),
    ("erase sign flipped",
     "Si[j] = a * Si[j] - a * b * w * k[j]", "Si[j] = a * Si[j] + a * b * w * k[j]"),
    ("write sign flipped", "+ b * v[i] * k[j];", "- b * v[i] * k[j];"),
    ("state read along q", "w += Si[j] * k[j];", "w += Si[j] * q[j];"),
    ("read-out along k", "oi += Si[j] * q[j];", "oi += Si[j] * k[j];"),
    ("read-out before the update",
     "    double w = 0.0;\n    for (int j = 0; j < d_k; ++j) w += Si[j] * k[j];\n",
     "    double w = 0.0;\n    for (int j = 0; j < d_k; ++j) w += Si[j] * k[j];\n"
     "    { double oo = 0.0; for (int j = 0; j < d_k; ++j) oo += Si[j] * q[j];"
     " o[i] = oo; }\n    if (0)\n"),
    ("write uses the query",
     "+ b * v[i] * k[j];", "+ b * v[i] * q[j];"),
    ("softplus without its linear part",
     "return fmax(x, 0.0) + log1p(exp(-fabs(x)));",
     "return log1p(exp(-fabs(x)));"),
    ("A_log used without exp",
     "*a = exp(-exp(A_log) * oracle_softplus(g + dt_bias));",
     "*a = exp(-A_log * oracle_softplus(g + dt_bias));"),
    ("dt_bias dropped",
     "*a = exp(-exp(A_log) * oracle_softplus(g + dt_bias));",
     "*a = exp(-exp(A_log) * oracle_softplus(g));"),
    ("sigmoid sign flipped",
     "return 1.0 / (1.0 + exp(-x));", "return 1.0 / (1.0 + exp(x));"),
    ("direct decay not exponentiated", "*a = exp(g);", "*a = 1.0 + g;"),
    ("key head taken modulo",
     "    const int hk = h / group;\n", "    const int hk = h % h_k;\n"),
    ("decode key head taken modulo",
     "hk = h / group;\n    double a, b;", "hk = h % h_k;\n    double a, b;"),
    ("initial state ignored",
     "S0 ? S0[(size_t)i * d_k + j] : 0.0", "0.0"),
    ("sequence start ignored",
     "for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t)",
     "for (int64_t t = 0; t < cu_seqlens[n + 1]; ++t)"),
    ("tail eps outside the root",
     "1.0 / sqrt(ss / d + eps)", "1.0 / (sqrt(ss / d) + eps)"),
    ("tail sum instead of mean", "1.0 / sqrt(ss / d + eps)",
     "1.0 / sqrt(ss + eps)"),
    ("tail weight dropped", "xr[i] * inv_rms * w[i]", "xr[i] * inv_rms"),
    ("tail sigmoid instead of SiLU",
     "zr[i] * oracle_sigmoid(zr[i])", "oracle_sigmoid(zr[i])"),
    ("tail missing the root", "1.0 / sqrt(ss / d + eps)", "1.0 / (ss / d + eps)"),
]


def _build(tmp_path, idx, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor must match exactly once: %r" % old
    path = os.path.join(str(tmp_path), "m%d.c" % idx)
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(str(tmp_path), "libm%d.so" % idx)
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o",
                           lib, path, "-lm"])
    return lib


@pytest.mark.parametrize("idx", range(len(MUTANTS)),
                         ids=[m[0].replace(" ", "_") for m in MUTANTS])
def test_mutant_is_caught(tmp_path, idx):
    name, old, new = MUTANTS[idx]
    lib = _build(tmp_path, idx, old, new)
    caught = []
    with O.use_library(lib):
        for pin in P.ALL_PINS:
            try:
                pin()
            except AssertionError:
                caught.append(pin.__name__)
    assert caught, "mutant '%s' passed every pin" % name
