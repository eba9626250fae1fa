"""Pins of the oracle where the shrink is live (W_e != 0), and of its reconstruction MSE.

The shrink regime has no closed form, so the oracle is compared trace for trace with an
independent exact re-statement of the iteration (`tests/exact_ref.py`): exact rationals,
the binary32 rounding of s, z and beta done by exact nearest-even selection, and |r|^(p-1)
in 60-digit decimal arithmetic. It fixes the order the techreport gives
["Outlier-aware optimization without gradients"]: sub-problem 1 (generalized soft-threshold
of the accepted iterate's residual with beta_t = beta0 * kappa^(t-1)), then sub-problem 2
(zero update with W_e), then beta <- beta * kappa ["Benchmark results / Llama-2":
p = 0.7, kappa = 1.01, 20 iterations, early stopping].
"""
from fractions import Fraction as F
import os

import numpy as np
import pytest

import synth
from tests.exact_ref import exact_solve

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mse_cases.txt")


def synth_w16(rows, cols, seed):
    return synth.half_bits(synth.student_t_weights(rows, cols, seed)).reshape(-1)


# (nbits, g, params, weight multiplier): beta0 = 1e4 makes the shrink move most residuals in
# every iteration; the last case keeps the pages' beta0 = 1 and scales the weights up, so
# only groups holding an outlier reach the shrink.
SHRINK_CASES = [
    (4, 64, dict(p=1.0, beta0=1e4), 1),
    (4, 64, dict(p=0.7, beta0=1e4), 1),
    (4, 64, dict(p=0.5, beta0=1e4), 1),
    (2, 16, dict(p=0.7, beta0=1e4), 1),
    (3, 64, dict(p=0.7, beta0=3e3, kappa=1.05), 1),
    (8, 32, dict(p=0.7, beta0=1e6), 1),
    (4, 64, dict(p=0.7, beta0=1.0), 100),
]


def case_groups(nbits, g, mult, n, seed):
    w = synth_w16(1, g * n, seed)
    if mult != 1:
        x = w.view(np.float16).astype(np.float32) * np.float32(mult)
        w = x.astype(np.float16).view(np.uint16)
    return [w[i * g:(i + 1) * g].view(np.float16) for i in range(n)]


@pytest.mark.parametrize("nbits,g,params,mult", SHRINK_CASES)
def test_active_shrink_trace_matches_exact(O, nbits, g, params, mult):
    if mult == 1:
        groups = case_groups(nbits, g, mult, 14, 7000 + nbits + g)
    else:
        # Keep groups whose range exceeds 2 * qmax * beta0^(-1/(2-p)) = 30: their largest
        # residual, up to half a step (range / 30), can leave the dead zone.
        groups = [x for x in case_groups(nbits, g, mult, 3000, 7000 + nbits + g)
                  if np.ptp(x.astype(np.float32)) > 30][:8]
        assert len(groups) >= 4
    active = 0
    for i, xg in enumerate(groups):
        what, act = group_mismatch(O, xg, nbits, params)
        assert what is None, f"group {i}: {what} differs from the exact iteration"
        active += act
    assert active >= (2 if mult != 1 else 5 * len(groups))


def group_mismatch(O, xg, nbits, params):
    """Compares the oracle's solve of one group with the exact iteration. Returns (what
    differs or None, number of iterations whose shrink moved some residual)."""
    ex_params = dict(params)
    beta0 = ex_params.pop("beta0", 1.0)
    ex = exact_solve(xg, nbits, shrink=True, beta0=beta0, **ex_params)
    got = O.solve_group(xg.astype(np.float64), nbits, beta=beta0, **ex_params)
    if len(got["trace_S"]) != len(ex["trace"]):
        return "evaluation count", ex["active"]
    for k, ((S_ex, acc_ex), S, acc) in enumerate(zip(ex["trace"], got["trace_S"],
                                                     got["trace_acc"])):
        if F(float(S)) != S_ex:         # the oracle's binary64 S holds the exact sum
            return f"S of evaluation {k}", ex["active"]
        if bool(acc) != acc_ex:
            return f"accept flag of evaluation {k}", ex["active"]
    if not np.array_equal(got["codes"], ex["codes"]):
        return "codes", ex["active"]
    if got["s"] != ex["s"] or got["z"] != ex["z"]:
        return "scale or zero", ex["active"]
    if got["shrink_active"] != (ex["active"] > 0):
        return "shrink-active flag", ex["active"]
    return None, ex["active"]


def test_active_shrink_without_early_stop(O):
    """Without early stopping every iterate is accepted and all iterations run."""
    for xg in case_groups(4, 64, 1, 4, 515):
        what, act = group_mismatch(O, xg, 4, dict(p=0.7, beta0=1e4, early_stop=0))
        assert what is None, what
        assert act == 20


# ---------------------------------------------------------------------------------------
# The shrink on values where the generalized soft-threshold is exact by construction
# ---------------------------------------------------------------------------------------
def test_shrink_dyadic_closed_forms(O):
    """p = 0.5 and r = 4^k: |r|^(p-1) = 2^-k exactly, so with beta = 2^m the operator gives
    r - 2^(-k-m) (or 0 in the dead zone |r| <= beta^(-1/(2-p)) = 2^(-2m/3)); at p = 1 it is
    the soft-threshold r - 1/beta. Every value here is a binary64 number, so the oracle's
    binary64 result must equal it exactly."""
    for k in range(-12, 4):
        for m in range(0, 12):
            r, beta = 4.0 ** k, 2.0 ** m
            want = max(r - 2.0 ** (-k - m), 0.0)
            assert O.shrink(r, 0.5, beta) == want, (k, m)
            assert O.shrink(-r, 0.5, beta) == -want
            assert O.shrink(r, 1.0, beta) == max(r - 2.0 ** -m, 0.0)


# ---------------------------------------------------------------------------------------
# Reconstruction MSE on cases worked by hand
# ---------------------------------------------------------------------------------------
def read_mse_cases():
    cases, cur = [], {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                if not line and cur:
                    cases.append(cur)
                    cur = {}
                continue
            k, v = line.split(":", 1)
            cur[k.strip()] = v.strip()
    if cur:
        cases.append(cur)
    return cases


@pytest.mark.parametrize("case", read_mse_cases(), ids=lambda c: c["name"])
def test_mse_worked_examples(O, case):
    vals = lambda k, t: np.array([float(v) for v in case[k].split()], t)  # noqa: E731
    g, zb = int(case["g"]), int(case["zero_bits"])
    w16 = vals("w", np.float16).view(np.uint16)
    codes = vals("codes", np.float64).astype(np.uint8)
    scale = vals("scale", np.float16).view(np.uint16)
    if zb == 16:
        zero, meta = vals("zero", np.float16).view(np.uint16), None
    else:
        zero, meta = vals("zq", np.float64).astype(np.uint8), vals("meta", np.float16).view(np.uint16)
    got = O.mse(w16, codes, scale, zero, meta, g, zb)
    assert F(got) == F(case["expected"]), case["name"]
