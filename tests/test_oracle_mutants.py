"""The oracle's pins must catch plausible mistakes.  Each case plants one
mistake in a copy of cce_oracle.c (on the CPU), builds it, points the oracle
wrapper at the copy and runs the pins of test_oracle.py: at least one pin must
fail.  The unmodified source must pass them all."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "cce_oracle.c")

# (name, text in the source, replacement, occurrence index)
MUTANTS = [
    ("dH drops the one-hot term", "(v == y ? 1.0 : 0.0)", "0.0", 0),
    ("dE drops the one-hot term", "(v == y ? 1.0 : 0.0)", "0.0", 1),
    ("loss has the wrong sign", "loss[r] = l - z[y];", "loss[r] = z[y] - l;", 0),
    ("lse forgets the max shift", "const double l = m + log(s);", "const double l = log(s);", 0),
    ("dH accumulates h instead of e", "out[d] += g * e[d];", "out[d] += g * h[d];", 0),
    ("dE accumulates e instead of h", "out[d] += g * h[d];", "out[d] += g * e[d];", 0),
    ("loss indexes the wrong logit", "loss[r] = l - z[y];", "loss[r] = l - z[(y + 1) % V];", 0),
    ("dE keeps ignored rows", "if (y == ignore_index) continue;", ";", 0),
    ("dE uses row 0's lse", "exp(z - lse[i])", "exp(z - lse[0])", 0),
    ("dH uses row 0's dloss", "dloss[i] * (exp(z[v] - l)", "dloss[0] * (exp(z[v] - l)", 0),
    ("dot product skips the last feature", "for (int64_t k = 0; k < n; ++k)", "for (int64_t k = 0; k + 1 < n; ++k)", 0),
    ("mean logit divides by N", "key[v] = nvalid ? s / (double)nvalid : 0.0;", "key[v] = s / (double)N;", 0),
]

PINS = [
    lambda: pins.test_hand_worked_example(),
    lambda: pins.test_zero_classifier_closed_form(np.random.default_rng(1)),
    lambda: pins.test_equal_rows_closed_form(np.random.default_rng(2)),
    lambda: pins.test_single_class(),
    lambda: pins.test_shift_invariance(np.random.default_rng(3)),
    lambda: pins.test_gradient_rows_sum_to_zero(np.random.default_rng(4)),
    lambda: pins.test_ignored_rows_contribute_nothing(np.random.default_rng(5)),
    lambda: pins.test_finite_differences(),
    lambda: pins.test_against_torch_cross_entropy((33, 24, 257)),
    lambda: pins.test_mean_logit_identity(np.random.default_rng(6)),
]


def _replace_nth(text, old, new, n):
    start = -1
    for _ in range(n + 1):
        start = text.find(old, start + 1)
        assert start >= 0, f"mutation site {old!r} #{n} not found"
    return text[:start] + new + text[start + len(old):]


def _build(tmp_path, text, tag):
    src = tmp_path / f"m_{tag}.c"
    src.write_text(text)
    so = tmp_path / f"m_{tag}.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(src), "-lm"], check=True)
    return str(so)


def _failures():
    bad = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            bad += 1
    return bad


@pytest.mark.parametrize("name,old,new,n", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new, n):
    text = _replace_nth(open(SRC).read(), old, new, n)
    oracle.use_library(_build(tmp_path, text, str(abs(hash(name)))))
    try:
        assert _failures() > 0, f"no pin caught: {name}"
    finally:
        oracle.use_library(None)


def test_unmodified_source_passes(tmp_path):
    oracle.use_library(_build(tmp_path, open(SRC).read(), "orig"))
    try:
        assert _failures() == 0
    finally:
        oracle.use_library(None)
