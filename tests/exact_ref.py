"""Exact rational re-statement of the HQQ iteration, for pinning the oracle.

Written independently of the oracle's C code: Python Fractions, no floating point except
the binary32 rounding of the solver state, which is done here by exact nearest-even
selection. It covers the regime where the shrink output W_e is zero everywhere (the
auxiliary variable then drops out of the zero update).
"""
from __future__ import annotations

from fractions import Fraction as F

import numpy as np


def f32_round(v: F) -> F:
    """Correctly rounded (nearest, ties to even) binary32 value of the exact rational v."""
    if v == 0:
        return F(0)
    approx = np.float32(float(v))
    cands = {approx,
             np.nextafter(approx, np.float32(np.inf)),
             np.nextafter(approx, np.float32(-np.inf))}
    best = None
    for c in cands:
        d = abs(F(float(c)) - v)
        even = (int(np.array(c, np.float32).view(np.uint32)) & 1) == 0
        key = (d, not even)
        if best is None or key < best[0]:
            best = (key, c)
    return F(float(best[1]))


def round_half_even(v: F) -> int:
    return round(v)  # Fraction.__round__ rounds half to even


def exact_solve(x16: np.ndarray, nbits: int, iters: int = 20, early_stop: bool = True):
    """Reduced HQQ iteration (W_e = 0) in exact arithmetic with binary32 s and z.

    Returns codes, s, z, passes (evaluation count incl. the initial one, running on through
    exact fixed points as the literal loop does), and the list of (S, accepted)."""
    qmax = (1 << nbits) - 1
    xs = [F(float(v)) for v in np.asarray(x16, np.float16)]
    g = len(xs)
    mn, mx = min(xs), max(xs)
    # s and z0 are the binary32 results of the binary32 operations max-min, qmax/rng, -min*s.
    mn32, mx32 = f32_round(mn), f32_round(mx)
    rng = f32_round(mx32 - mn32)
    s = f32_round(F(qmax) / rng) if rng > 0 else F(1)
    z = f32_round(-(mn32 * s))
    sum_x = sum(xs)

    def evaluate(z):
        q = []
        S = F(0)
        for x in xs:
            u = x * s + z
            c = min(max(round_half_even(u), 0), qmax)
            q.append(c)
            S += abs(u - c)
        return q, S

    q, S_best = evaluate(z)
    trace = [(S_best, True)]
    visited = [z]
    passes = 1
    for _ in range(iters):
        z_new = f32_round((F(sum(q)) - s * sum_x) / g)
        q_new, S_new = evaluate(z_new)
        visited.append(z_new)
        passes += 1
        if early_stop and S_new > S_best:
            trace.append((S_new, False))
            break
        trace.append((S_new, True))
        z, q, S_best = z_new, q_new, S_new
    return dict(codes=np.array(q, np.uint8), s=float(s), z=float(z), passes=passes,
                trace=trace, visited=[float(v) for v in visited])


def shrink_surely_zero(x16: np.ndarray, nbits: int, s: float, zs, p: float, beta_max: float):
    """True when every residual r = x - (q - z)/s over the given zeros is certainly below the
    threshold beta^(-1/(2-p)) at which the generalized soft-threshold starts to move r (the
    largest beta gives the smallest threshold)."""
    qmax = (1 << nbits) - 1
    x = np.asarray(x16, np.float16).astype(np.float64)
    tau = beta_max ** (-1.0 / (2.0 - p))
    for z in zs:
        u = x * s + z
        q = np.clip(np.rint(u), 0, qmax)
        r = np.abs(u - q) / s
        if r.max() > tau * (1 - 1e-6):
            return False
    return True
