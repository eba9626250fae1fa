"""Pins of the CPU oracle against what the pages and mathematics fix (CPU only).

Each test names the part of the method it pins; together they are chosen so that a dropped
term, a wrong sign, a wrong index or a swapped operand anywhere in the oracle fails one.
"""
from fractions import Fraction as F

import numpy as np
import pytest

import synth
from tests.exact_ref import exact_solve, shrink_surely_zero

RNG = np.random.default_rng(12345)


def synth_w16(rows, cols, seed):
    return synth.half_bits(synth.student_t_weights(rows, cols, seed)).reshape(-1)


# ---------------------------------------------------------------------------------------
# binary16 conversion (used for the inputs and the stored scale/zero)
# ---------------------------------------------------------------------------------------
def test_half_to_float_all_patterns(O):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float32)
    got = np.array([O.half_to_float(int(h)) for h in pats], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_float_to_half_matches_numpy_rne(O):
    vals = np.concatenate([
        RNG.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        RNG.standard_normal(5000).astype(np.float32) * np.float32(1e-6),   # subnormal range
        np.float32(2.0) ** RNG.integers(-30, 17, 3000).astype(np.float32),
        np.array([65504, 65519.99, 65520, 65536, 1e9, -1e9, 2.0 ** -24, 2.0 ** -25,
                  3 * 2.0 ** -26, 2.0 ** -14, 0.0, -0.0, 1.0 + 2.0 ** -11,
                  1.0 + 3 * 2.0 ** -11], np.float32),
    ])
    # exact binary16 ties: midpoints between consecutive binary16 values
    h = RNG.integers(0, 0x7bff, 3000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    vals = np.concatenate([vals, ((lo + hi) / 2).astype(np.float32)])
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([O.float_to_half(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------------------
# Sub-problem 1: generalized soft-thresholding
# ---------------------------------------------------------------------------------------
def test_shrink_formula_odd_zero_and_threshold(O):
    for p, beta in [(0.7, 1.0), (0.7, 3.0), (0.5, 10.0), (0.9, 0.5)]:
        p32, b32 = float(np.float32(p)), float(np.float32(beta))
        tau = b32 ** (-1.0 / (2.0 - p32))
        for r in list(RNG.standard_normal(300) * 3) + [tau * 0.999, tau * 1.001, 1e-12]:
            got = O.shrink(r, p32, b32)
            a = abs(r)
            ref = np.sign(r) * max(a - a ** (p32 - 1.0) / b32, 0.0)
            assert got == pytest.approx(ref, rel=1e-12, abs=1e-300)
            assert O.shrink(-r, p32, b32) == -got                 # odd
            if a <= tau * (1 - 1e-9):
                assert got == 0.0                                 # dead zone
            if a >= tau * (1 + 1e-9):
                assert got != 0.0 and np.sign(got) == np.sign(r)  # moves toward 0, keeps sign
                assert abs(got) < a
        assert O.shrink(0.0, p32, b32) == 0.0                     # limit at r = 0


def test_shrink_p1_is_prox_of_abs(O):
    """At p = 1 the operator is the exact proximal map of |w|: argmin |w| + beta/2 (w - r)^2."""
    for beta in [0.5, 1.0, 4.0]:
        for r in RNG.standard_normal(40) * 2:
            grid = np.linspace(-5, 5, 200001)
            obj = np.abs(grid) + beta / 2 * (grid - r) ** 2
            w_star = grid[np.argmin(obj)]
            assert O.shrink(float(r), 1.0, beta) == pytest.approx(w_star, abs=1e-4)


# ---------------------------------------------------------------------------------------
# Sub-problem 2: the zero update is the closed-form minimiser
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("g", [2, 3, 5, 8, 16])
def test_zero_update_is_least_squares_minimiser(O, g):
    for _ in range(20):
        x = RNG.standard_normal(g) * 0.05
        we = RNG.standard_normal(g) * 0.01 * (RNG.random(g) < 0.5)
        s = float(np.float32(RNG.uniform(20, 200)))
        q = RNG.integers(0, 16, g).astype(np.float64)
        z = O.zero_update(x, q, we, s)
        obj = lambda zz: np.sum(((q - zz) / s - (x - we)) ** 2)  # noqa: E731
        grid = z + np.arange(-10000, 10001) * 1e-4
        vals = np.array([obj(v) for v in grid])
        k = np.argmin(vals)
        assert abs(grid[k] - z) <= 1e-4 + 1e-12
        assert obj(z) <= vals.min() + 1e-9


# ---------------------------------------------------------------------------------------
# Initialisation: iters = 0 is plain min-max round-to-nearest
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("nbits,g", [(1, 16), (2, 16), (3, 64), (4, 64), (4, 128), (8, 32)])
def test_iters0_is_minmax_rtn(O, nbits, g):
    w16 = synth_w16(64, 512, 7 + nbits)
    r = O.solve_groups(w16, g, nbits, iters=0)
    x = w16.view(np.float16).astype(np.float32).reshape(-1, g)
    qmax = np.float32((1 << nbits) - 1)
    mn, mx = x.min(1), x.max(1)
    rng = (mx - mn).astype(np.float32)
    s = np.where(rng > 0, qmax / np.where(rng > 0, rng, 1), 1).astype(np.float32)
    z = (-(mn * s)).astype(np.float32)
    u = x.astype(np.float64) * s[:, None].astype(np.float64) + z[:, None].astype(np.float64)
    q = np.clip(np.rint(u), 0, qmax).astype(np.uint8)
    assert np.array_equal(r["codes"], q.reshape(-1))
    assert np.array_equal(r["zero_f32"], z)
    assert np.array_equal(r["scale"], (np.float32(1) / s).astype(np.float16).view(np.uint16))
    assert np.all(r["passes"] == 1)


# ---------------------------------------------------------------------------------------
# Whole solver against the exact rational re-statement (W_e = 0 regime)
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("nbits,g,ngroups", [(4, 64, 60), (4, 128, 30), (2, 16, 150),
                                             (2, 32, 100), (3, 64, 60), (8, 16, 40),
                                             (1, 16, 60)])
def test_solver_equals_exact_rational_iteration(O, nbits, g, ngroups):
    w16 = synth_w16(1, g * ngroups, 1000 + 10 * nbits + g)
    r = O.solve_groups(w16, g, nbits)
    beta_max = float(np.float32(1.01)) ** 20
    checked = 0
    for i in range(ngroups):
        xg = w16[i * g:(i + 1) * g].view(np.float16)
        ex = exact_solve(xg, nbits)
        if not shrink_surely_zero(xg, nbits, ex["s"], ex["visited"], 0.7, beta_max):
            continue
        checked += 1
        assert np.array_equal(r["codes"][i * g:(i + 1) * g], ex["codes"]), i
        assert float(r["s"][i]) == ex["s"]
        assert float(r["zero_f32"][i]) == ex["z"], i
        assert int(r["passes"][i]) == ex["passes"], i
        assert r["shrink_active"][i] == 0
    assert checked >= ngroups * 0.9


def test_exact_iteration_trace_matches(O):
    """Every evaluation's exact error S = sum |x*s + z - q| and its accept flag agree."""
    w16 = synth_w16(1, 64 * 40, 4242)
    for i in range(40):
        xg = w16[i * 64:(i + 1) * 64].view(np.float16)
        ex = exact_solve(xg, 4)
        got = O.solve_group(xg.astype(np.float64), 4)
        assert len(got["trace_S"]) == len(ex["trace"])
        for (S_ex, acc_ex), S, acc in zip(ex["trace"], got["trace_S"], got["trace_acc"]):
            assert F(float(S)) == S_ex      # binary64 held the exact sum
            assert bool(acc) == acc_ex


# ---------------------------------------------------------------------------------------
# Invariants of the iteration
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("beta", [1.0, 1e4])
def test_accepted_error_never_rises(O, beta):
    """Accepted errors are non-increasing, the result is no worse than RTN, and a stop is
    always caused by a strictly larger error. beta = 1e4 makes the shrink active."""
    w16 = synth_w16(4, 1024, 99)
    active = 0
    for i in range(64):
        x = w16[i * 64:(i + 1) * 64].view(np.float16).astype(np.float64)
        t = O.solve_group(x, 4, beta=beta)
        S, acc = t["trace_S"], t["trace_acc"].astype(bool)
        accepted = S[acc]
        assert np.all(np.diff(accepted) <= 0)
        assert accepted[-1] <= S[0]
        if not acc[-1]:
            assert S[-1] > accepted[-1]
            assert acc[:-1].all()
        else:
            assert t["passes"] == 21
        active += t["shrink_active"]
    if beta > 1:
        assert active > 0


def test_codes_in_range_all_bits(O):
    for nbits in (1, 2, 3, 4, 8):
        w16 = synth_w16(8, 256, 5 + nbits)
        r = O.solve_groups(w16, 32, nbits)
        assert r["codes"].max() <= (1 << nbits) - 1


def test_special_groups(O):
    # constant group: s = 1, z = -x, all codes 0, exact reconstruction
    for v in (0.0, 0.125, -3.5):
        x = np.full(32, v)
        t = O.solve_group(x, 4)
        assert np.all(t["codes"] == 0) and t["s"] == 1.0 and t["z"] == -v + 0.0
        assert t["err"] == 0.0
    # two-valued group: codes only 0 and qmax; the min-max start is already exact
    for nbits in (2, 4):
        x = np.where(RNG.random(64) < 0.5, -0.0625, 0.1875)
        x[0], x[1] = -0.0625, 0.1875
        t = O.solve_group(x, nbits)
        assert set(np.unique(t["codes"])) == {0, (1 << nbits) - 1}
        assert t["err"] == 0.0


def test_scale_equivariance(O):
    """W * 2^k leaves codes and zero unchanged and multiplies the stored scale by 2^k
    (checked where the shrink stays inactive for both inputs)."""
    w16 = synth_w16(8, 512, 31)
    base = O.solve_groups(w16, 64, 4)
    x = w16.view(np.float16).astype(np.float32)
    for k in (1, 3):
        xs = (x * np.float32(2.0 ** k)).astype(np.float16)
        assert np.array_equal(xs.astype(np.float32), x * np.float32(2.0 ** k))
        r = O.solve_groups(xs.view(np.uint16), 64, 4)
        ok = (r["shrink_active"] == 0) & (base["shrink_active"] == 0)
        assert ok.mean() > 0.9
        cg = np.repeat(ok, 64)
        assert np.array_equal(r["codes"][cg], base["codes"][cg])
        assert np.array_equal(r["zero_f32"][ok], base["zero_f32"][ok])
        sc = base["scale"].view(np.float16).astype(np.float32)[ok] * np.float32(2.0 ** k)
        assert np.array_equal(r["scale"].view(np.float16).astype(np.float32)[ok], sc)


def test_literal_iteration_continues_through_fixed_points(O):
    """A tie is not a rise: a group whose zero stops changing keeps being accepted until the
    iteration budget is used up."""
    w16 = synth_w16(2, 4096, 77)
    r = O.solve_groups(w16, 64, 4)
    fixed = r["passes"] == 21
    assert fixed.mean() > 0.3
    assert np.all(r["last_change"][fixed] <= 20)


# ---------------------------------------------------------------------------------------
# Zero-point 8-bit storage, dequantization, MSE
# ---------------------------------------------------------------------------------------
def test_zero_requant_range_and_roundtrip(O):
    z = (RNG.standard_normal(5000) * 3 + 7).astype(np.float32)
    zq, meta = O.zero_requant(z)
    assert zq.min() == 0 and zq.max() == 255
    assert zq[np.argmin(z)] == 0 and zq[np.argmax(z)] == 255
    step = float(meta[0:1].view(np.float16)[0])
    base = float(meta[1:2].view(np.float16)[0])
    assert step == float(np.float16((z.max() - z.min()) / np.float32(255)))
    assert base == float(np.float16(z.min()))
    zr = zq.astype(np.float64) * step + base
    inner = (zq > 0) & (zq < 255)
    assert np.max(np.abs(zr - z)[inner]) <= 0.5 * step * (1 + 1e-5)   # half a step inside
    assert np.max(np.abs(zr - z)) <= (0.5 + 255 * 2.0 ** -11) * step + abs(base - z.min())
    # each code is the nearest grid point
    for k in RNG.integers(0, z.size, 200):
        d = np.abs(np.arange(256) * step + base - z[k])
        assert abs(d[zq[k]] - d.min()) <= 1e-6 * step
    # constant zeros: step 1, everything at the base
    zq, meta = O.zero_requant(np.full(10, 3.25, np.float32))
    assert np.all(zq == 0) and meta[1:2].view(np.float16)[0] == 3.25
    assert meta[0:1].view(np.float16)[0] == 1.0


def test_dequantize_identity_and_formula(O):
    for nbits in (1, 2, 3, 4, 8):
        n = 640
        codes = RNG.integers(0, 1 << nbits, n).astype(np.uint8)
        ones = np.full(n // 64, np.float16(1.0)).view(np.uint16)
        zeros = np.zeros(n // 64, np.uint16)
        out = O.dequantize(codes, ones, zeros, None, 64, 16)
        assert np.array_equal(out.view(np.float16).astype(np.float32), codes.astype(np.float32))
    codes = RNG.integers(0, 16, 256).astype(np.uint8)
    scale = (RNG.random(4) * 0.01 + 0.001).astype(np.float16)
    zero = (RNG.random(4) * 15).astype(np.float16)
    out = O.dequantize(codes, scale.view(np.uint16), zero.view(np.uint16), None, 64, 16)
    ref = ((codes.astype(np.float32) - np.repeat(zero.astype(np.float32), 64))
           * np.repeat(scale.astype(np.float32), 64)).astype(np.float16)
    assert np.array_equal(out, ref.view(np.uint16))
    zq = RNG.integers(0, 256, 4).astype(np.uint8)
    meta = np.array([0.05, 2.0], np.float16)
    out = O.dequantize(codes, scale.view(np.uint16), zq, meta.view(np.uint16), 64, 8)
    zf = (zq.astype(np.float64) * np.float64(meta[0]) + np.float64(meta[1])).astype(np.float32)
    ref = ((codes.astype(np.float32) - np.repeat(zf, 64))
           * np.repeat(scale.astype(np.float32), 64)).astype(np.float16)
    assert np.array_equal(out, ref.view(np.uint16))


def test_mse_definition(O):
    w16 = synth_w16(4, 256, 3)
    r = O.quantize(w16, 64, 4)
    mse = O.mse(w16, r["codes"], r["scale"], r["zero"], None, 64, 16)
    x = w16.view(np.float16).astype(np.float32)
    sc = np.repeat(r["scale"].view(np.float16).astype(np.float32), 64)
    zf = np.repeat(r["zero"].view(np.float16).astype(np.float32), 64)
    res = x - (r["codes"].astype(np.float32) - zf) * sc
    assert mse == pytest.approx(np.mean(res.astype(np.float64) ** 2), rel=1e-12)
    # the solver improves on round-to-nearest
    r0 = O.quantize(w16, 64, 4, iters=0)
    mse0 = O.mse(w16, r0["codes"], r0["scale"], r0["zero"], None, 64, 16)
    assert mse < mse0 * 1.02
