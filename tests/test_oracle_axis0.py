"""Pins of the oracle's axis-0 grouping (groups of g consecutive elements down a column),
CPU only. The grouping reading: group (b, j) is W[b*g:(b+1)*g, j]; per-group outputs form a
[rows/g, cols] row-major array; codes keep the tensor's row-major order. Pinned by closed
forms, by the independent exact rational iteration on column runs, and by the layout of
per-group values in the reconstruction."""
import numpy as np
import pytest

import synth
from tests.exact_ref import exact_solve, shrink_surely_zero

RNG = np.random.default_rng(99)


def f16(a):
    return np.asarray(a, np.float16)


def test_axis0_min_max_closed_form(O):
    # iters = 0 is min-max round-to-nearest. Two row blocks of 16 rows, four columns:
    # a ramp (codes 0..15, scale 1/16, zero 0), a constant (s = 1, z = -0.5, code 0), the
    # reversed ramp, and a ramp offset by 1 (s = 16, z = -16). Block 1 holds the same
    # columns scaled by 2 (scale 1/8).
    g, rows, cols = 16, 32, 4
    ramp = np.arange(16) / 16
    w = np.zeros((rows, cols))
    w[:16, 0], w[:16, 1], w[:16, 2], w[:16, 3] = ramp, 0.5, ramp[::-1], ramp + 1
    w[16:] = 2 * w[:16]
    w16 = f16(w)
    assert np.array_equal(w16.astype(np.float64), w)          # exact in binary16
    r = O.quantize_axis0(w16.view(np.uint16).reshape(-1), rows, cols, g, 4, iters=0)
    codes = r["codes"].reshape(rows, cols)
    k = np.arange(16)
    for b in range(2):
        blk = codes[16 * b:16 * (b + 1)]
        assert np.array_equal(blk[:, 0], k) and np.array_equal(blk[:, 2], k[::-1])
        assert np.all(blk[:, 1] == 0) and np.array_equal(blk[:, 3], k)
    scale = r["scale"].view(np.float16).reshape(2, cols).astype(np.float64)
    zero = r["zero"].view(np.float16).reshape(2, cols).astype(np.float64)
    assert scale[0].tolist() == [1 / 16, 1.0, 1 / 16, 1 / 16]
    assert scale[1].tolist() == [1 / 8, 1.0, 1 / 8, 1 / 8]
    assert zero[0].tolist() == [0.0, -0.5, 0.0, -16.0]
    assert zero[1].tolist() == [0.0, -1.0, 0.0, -16.0]
    back = O.dequantize_axis0(r["codes"], r["scale"], r["zero"], None, rows, cols, g, 16)
    assert np.array_equal(back, w16.view(np.uint16).reshape(-1))   # every value on its grid


@pytest.mark.parametrize("nbits,g", [(4, 64), (2, 16), (3, 32)])
def test_axis0_column_runs_equal_exact_iteration(O, nbits, g):
    # each column run solved by the exact rational re-statement (no oracle code involved)
    rows, cols = 2 * g, 24
    w16 = synth.half_bits(synth.student_t_weights(rows, cols, 500 + g)).reshape(rows, cols)
    r = O.quantize_axis0(w16.reshape(-1), rows, cols, g, nbits)
    codes = r["codes"].reshape(rows, cols)
    z = r["zero_f32"].reshape(rows // g, cols)
    passes = r["passes"].reshape(rows // g, cols)
    beta_max = float(np.float32(1.01)) ** 20
    checked = 0
    for b in range(rows // g):
        for j in range(cols):
            xg = w16[b * g:(b + 1) * g, j].view(np.float16)
            ex = exact_solve(xg, nbits)
            if not shrink_surely_zero(xg, nbits, ex["s"], ex["visited"], 0.7, beta_max):
                continue
            checked += 1
            assert np.array_equal(codes[b * g:(b + 1) * g, j], ex["codes"]), (b, j)
            assert float(z[b, j]) == ex["z"] and int(passes[b, j]) == ex["passes"], (b, j)
            assert float(np.float16(1.0 / np.float32(ex["s"]))) == \
                float(r["scale"].view(np.float16).reshape(rows // g, cols)[b, j])
    assert checked >= 0.9 * (rows // g) * cols


def test_axis0_reconstruction_uses_the_right_group(O):
    # codes 1, zeros 0 and a distinct power of two as each group's scale: every element
    # reads back exactly its own group's scale
    g, rows, cols = 16, 48, 5
    nb = rows // g
    scale = f16(2.0 ** -np.arange(nb * cols).reshape(nb, cols))
    codes = np.ones(rows * cols, np.uint8)
    zero = np.zeros(nb * cols, np.uint16)
    back = O.dequantize_axis0(codes, scale.view(np.uint16).reshape(-1), zero, None, rows, cols,
                              g, 16).view(np.float16).reshape(rows, cols)
    assert np.array_equal(back, np.repeat(scale, g, axis=0))


def test_axis0_eight_bit_zero_layout(O):
    # the 8-bit zero grid is per tensor; each stored code reads back within half a step of
    # its own group's binary32 zero
    g, rows, cols = 32, 96, 40
    w16 = synth.half_bits(synth.student_t_weights(rows, cols, 77)).reshape(-1)
    r = O.quantize_axis0(w16, rows, cols, g, 4, zero_bits=8)
    step = float(r["zero_meta"][0:1].view(np.float16)[0])
    base = float(r["zero_meta"][1:2].view(np.float16)[0])
    zr = r["zero"].astype(np.float64) * step + base
    z = r["zero_f32"].astype(np.float64)
    assert np.all(np.abs(zr - z) <= (0.5 + 255 * 2.0 ** -11) * step + abs(base - z.min()))
    assert zr.shape == (rows // g * cols,)
