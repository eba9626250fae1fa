"""Pins of the oracle's quantized linear layer Y = X · W_r^T (CPU only): exact sums by brute
force in rational arithmetic, the orientation of W_r (one-hot inputs read single weights back),
and the group lookup of the reconstruction it uses."""
from fractions import Fraction as F

import numpy as np
import pytest

import synth

RNG = np.random.default_rng(5150)


def quantized(O, n, k, g, nbits, zero_bits, seed):
    w16 = synth.half_bits(synth.student_t_weights(n, k, seed)).reshape(-1)
    return O.quantize(w16, g, nbits, zero_bits=zero_bits)


@pytest.mark.parametrize("nbits,g,zero_bits", [(4, 16, 16), (2, 32, 8), (3, 16, 16), (8, 16, 8)])
def test_gemm_equals_exact_sum(O, nbits, g, zero_bits):
    m, n, k = 3, 5, 32
    r = quantized(O, n, k, g, nbits, zero_bits, 60 + nbits)
    x = (RNG.integers(-64, 64, m * k) / 64).astype(np.float16)      # dyadic: sums stay exact
    y = O.gemm(x.view(np.uint16), r["codes"], r["scale"], r["zero"], r["zero_meta"], n, k, g,
               zero_bits)
    w = O.dequantize(r["codes"], r["scale"], r["zero"], r["zero_meta"], g, zero_bits)
    w = w.view(np.float16).reshape(n, k)
    for i in range(m):
        for j in range(n):
            exact = sum(F(float(x[i * k + t])) * F(float(w[j, t])) for t in range(k))
            assert F(float(y[i, j])) == exact, (i, j)


def test_gemm_orientation(O):
    # a one-hot row of X picks one column of W_r: Y[i, j] = W_r[j, t_i]
    n, k, g = 7, 64, 16
    r = quantized(O, n, k, g, 4, 16, 11)
    w = O.dequantize(r["codes"], r["scale"], r["zero"], r["zero_meta"], g, 16)
    w = w.view(np.float16).astype(np.float64).reshape(n, k)
    t = [0, 5, 17, 63]
    x = np.zeros((len(t), k), np.float16)
    x[np.arange(len(t)), t] = 1.0
    y = O.gemm(x.view(np.uint16), r["codes"], r["scale"], r["zero"], r["zero_meta"], n, k, g, 16)
    assert np.array_equal(y, w[:, t].T)
