"""Pins of the oracle's rounding order on binary16 ties, CPU only. The reconstruction rounds
the binary32 result to binary16 (two roundings); on the tie cases of tests/ties.py the single
rounding of the exact value gives the other binary16 neighbour, so these cases tell the two
orders apart. Expected values here come from exact rational arithmetic, not the oracle."""
from fractions import Fraction as F

import numpy as np

from tests import ties

STEP, BASE = 0.0633, -1.014


def f32(x: F) -> F:
    """Round a rational to binary32 (nearest even), through binary64 when that is exact."""
    d = float(x)
    assert F(d) == x, "operand not exact in binary64"
    return F(float(np.float32(d)))


def f16(x: F) -> np.float16:
    d = float(x)
    assert F(d) == x
    return np.float16(d)


def test_dequantize_rounds_to_binary32_first(O):
    q, zq, s = ties.dequant_ties(64, 11, STEP, BASE)
    g, n = 16, q.size
    meta = np.array([np.float16(STEP), np.float16(BASE)]).view(np.uint16)
    codes = np.repeat(q, g)                      # every element of group i is a tie case
    out = O.dequantize(codes, s.view(np.uint16), zq, meta, g, 8).view(np.float16)
    st, bs = F(float(np.float16(STEP))), F(float(np.float16(BASE)))
    for i in range(n):
        zf = f32(int(zq[i]) * st + bs)
        d = f32(int(q[i]) - zf)
        prod = d * F(float(s[i]))
        assert out[i * g] == f16(f32(prod)), i
        assert out[i * g] != f16(prod), i        # the other order would differ here
        assert np.all(out[i * g:(i + 1) * g] == out[i * g])


def test_scale_dequant_rounds_to_binary32_first(O):
    q, st, bs = ties.scale_dequant_ties(32, 12)
    group = 8                                    # one tie triple per run of 8 scales
    meta = np.stack([st, bs], axis=1).reshape(-1).view(np.uint16)
    codes = np.repeat(q, group)
    out = O.scale_dequant(codes, meta, group=group).view(np.float16)
    for i in range(q.size):
        exact = int(q[i]) * F(float(st[i])) + F(float(bs[i]))
        assert out[i * group] == f16(f32(exact)), i
        assert out[i * group] != f16(exact), i
