"""Exact re-statement of the HQQ iteration, for pinning the oracle.

Written independently of the oracle's C code: Python Fractions, no floating point except
the binary32 rounding of the solver state (scale, zero, beta), which is done here by exact
nearest-even selection. Two regimes:

* the reduced iteration, where the shrink output W_e is zero everywhere and the auxiliary
  variable drops out of the zero update (``shrink=False``);
* the full iteration with a live shrink (``shrink=True``): sub-problem 1 of techreport.ngo
  "Half-Quadratic Quantization of Large Machine Learning Models", section "Outlier-aware
  optimization without gradients" -- the generalized soft-threshold
  W_e = sign(r) * max(|r| - |r|^(p-1)/beta, 0) of the residual r = W - W_r of the accepted
  iterate -- then sub-problem 2, z = mean(q - (W - W_e) * s), then beta <- beta * kappa (the
  parameters of its section "Benchmark results / Llama-2"). Every quantity is an exact
  rational except |r|^(p-1) for p != 1, which is evaluated in 60-digit decimal arithmetic
  (correctly rounded at that precision), about 40 digits beyond anything binary32 or binary64
  can resolve.
"""
from __future__ import annotations

import decimal
from fractions import Fraction as F

import numpy as np

_DEC = decimal.Context(prec=60, rounding=decimal.ROUND_HALF_EVEN)


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


def _dec(v: F) -> decimal.Decimal:
    return _DEC.divide(decimal.Decimal(v.numerator), decimal.Decimal(v.denominator))


def power(a: F, e: F) -> F:
    """a**e for a > 0: exact when e == 0, else 60-digit decimal arithmetic."""
    if e == 0:
        return F(1)
    return F(_DEC.power(_dec(a), _dec(e)))


def soft_threshold(r: F, p: F, beta: F) -> F:
    """Generalized soft-threshold sign(r) * max(|r| - |r|^(p-1)/beta, 0); 0 at r = 0 (the
    operator's limit for p < 1)."""
    if r == 0:
        return F(0)
    a = abs(r)
    m = a - power(a, p - 1) / beta
    if m <= 0:
        return F(0)
    return m if r > 0 else -m


def exact_solve(x16: np.ndarray, nbits: int, iters: int = 20, early_stop: bool = True,
                shrink: bool = False, p: float = 0.7, beta0: float = 1.0,
                kappa: float = 1.01):
    """The HQQ iteration for one group in exact arithmetic with binary32 s, z and beta.

    shrink=False: the reduced iteration (W_e = 0). shrink=True: the full iteration with the
    generalized soft-threshold of the accepted iterate's residual, beta_t = beta0 * kappa^(t-1)
    as a sequence of binary32 products, multiplied after the zero update.

    Returns codes, s, z, passes (evaluation count incl. the initial one, running on through
    exact fixed points as the literal loop does), trace (list of (S, accepted)), the zeros
    visited, and `active` (number of iterations whose W_e had a non-zero entry)."""
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
    p32 = F(float(np.float32(p)))
    kappa32 = F(float(np.float32(kappa)))
    beta = F(float(np.float32(beta0)))

    def evaluate(z):
        q, e = [], []
        for x in xs:
            u = x * s + z
            c = min(max(round_half_even(u), 0), qmax)
            q.append(c)
            e.append(u - c)
        return q, e, sum(abs(v) for v in e)

    q, e, S_best = evaluate(z)
    trace = [(S_best, True)]
    visited = [z]
    passes, active = 1, 0
    for _ in range(iters):
        if shrink:
            # residual of the accepted iterate: r = x - (q - z)/s = (x*s + z - q)/s
            we = [soft_threshold(ej / s, p32, beta) for ej in e]
            active += any(w != 0 for w in we)
            z_new = f32_round(sum(qj - (xj - wj) * s for qj, xj, wj in zip(q, xs, we)) / g)
            beta = f32_round(beta * kappa32)
        else:
            z_new = f32_round((F(sum(q)) - s * sum_x) / g)
        q_new, e_new, S_new = evaluate(z_new)
        visited.append(z_new)
        passes += 1
        if early_stop and S_new > S_best:
            trace.append((S_new, False))
            break
        trace.append((S_new, True))
        z, q, e, S_best = z_new, q_new, e_new, S_new
    return dict(codes=np.array(q, np.uint8), s=float(s), z=float(z), passes=passes,
                trace=trace, visited=[float(v) for v in visited], active=active)


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
