"""The oracle's pins catch plausible mistakes: each test plants one mistake in a copy of the
oracle's C source (on the CPU, in a temporary directory), builds it, and checks that the
pins of the solver reject it. The oracle itself is never modified.

The mistakes are local edits of the steps of techreport.ngo "Half-Quadratic Quantization of
Large Machine Learning Models", section "Outlier-aware optimization without gradients"
(shrink of the residual, zero update, beta schedule) and of the early-stop rule of its
section "Benchmark results / Llama-2".

One reading needs no mutation of its own: feeding the shrink the candidate's residual
instead of the accepted one. In the oracle's loop a candidate is either accepted (its
residual becomes the accepted one) or ends the loop, so both readings compute the same
iteration; a stale residual (the accepted one not carried forward) is the mistake that
differs, and it is planted below.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle.hqq_oracle import CFLAGS, Oracle
from tests.exact_ref import exact_solve
from tests.test_oracle_shrink import case_groups, group_mismatch

SRC = os.path.join(os.path.dirname(oracle.__file__), "hqq_oracle.c")

KAPPA_LINE = "        beta = beta * kappa;\n"
LOOP_HEAD = "    for (int t = 1; t <= iters; ++t) {\n"

MUTATIONS = {
    "kappa applied before the shrink": [
        (KAPPA_LINE, ""), (LOOP_HEAD, LOOP_HEAD + KAPPA_LINE)],
    "beta never multiplied by kappa": [(KAPPA_LINE, "")],
    "stale residual (accepted residual not carried forward)": [
        ("        memcpy(r, rn, sizeof(double) * (size_t)g);\n", "")],
    "residual with the wrong sign": [
        ("        r[j] = d / (double)s;", "        r[j] = -d / (double)s;")],
    "W_e added instead of subtracted in the zero update": [
        ("double target = x[j] - we[j];", "double target = x[j] + we[j];")],
    "W_e not scaled by s in the zero update": [
        ("double term = q[j] - target * (double)s;",
         "double term = q[j] - x[j] * (double)s + we[j];")],
    "shrink exponent p instead of p - 1": [
        ("pow(a, (double)p - 1.0)", "pow(a, (double)p)")],
    "shrink multiplies by beta": [
        ("pow(a, (double)p - 1.0) / (double)beta", "pow(a, (double)p - 1.0) * (double)beta")],
    "a tie stops the iteration": [
        ("if (early_stop && S_new > S_best)", "if (early_stop && S_new >= S_best)")],
    "zero update averaged over g + 1": [
        ("return (float)(acc / (double)g);", "return (float)(acc / (double)(g + 1));")],
}


def build_mutant(tmp_path, edits):
    src = open(SRC).read()
    for old, new in edits:
        assert src.count(old) == 1, f"mutation site not unique: {old!r}"
        src = src.replace(old, new)
    c = os.path.join(tmp_path, "mutant.c")
    so = os.path.join(tmp_path, "libmutant.so")
    with open(c, "w") as f:
        f.write(src)
    subprocess.check_call(["gcc", *CFLAGS, "-o", so, c, "-lm"])
    return Oracle(so)


def pins_reject(M) -> str | None:
    """Runs the solver pins on a few groups; returns what they caught, or None."""
    for params in (dict(p=0.7, beta0=1e4), dict(p=1.0, beta0=1e4)):
        for xg in case_groups(4, 64, 1, 3, 7068):
            what, _ = group_mismatch(M, xg, 4, params)
            if what is not None:
                return f"active shrink ({params}): {what}"
    # the reduced iteration (no shrink): the exact trace, ties included
    w = case_groups(4, 64, 1, 24, 4242)
    for xg in w:
        ex = exact_solve(xg, 4)
        got = M.solve_group(xg.astype(np.float64), 4)
        if got["passes"] != ex["passes"] or not np.array_equal(got["codes"], ex["codes"]) \
                or got["z"] != ex["z"]:
            return "reduced iteration"
    return None


def test_unmutated_oracle_passes(tmp_path):
    assert pins_reject(build_mutant(str(tmp_path), [])) is None


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(tmp_path, name):
    M = build_mutant(str(tmp_path), MUTATIONS[name])
    assert pins_reject(M) is not None, f"planted mistake not caught: {name}"
