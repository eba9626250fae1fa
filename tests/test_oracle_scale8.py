"""Pins of the oracle's 8-bit scales (CPU only).

The pages' HQQ_g16_s variant stores its per-group scales on 8-bit grids, one per 128 scales
[techreport.ngo, "Half-Quadratic Quantization of Large Machine Learning Models", section
"Benchmark results / Llama-2", note on the HQQ_g16_s row]. The reading (min-max affine uint8
round-to-nearest per group of scales, like the 8-bit zero-point) is pinned here against
exact grids, exact-arithmetic nearest codes, the half-step error bound and the grouping.
"""
from fractions import Fraction as F

import numpy as np

RNG = np.random.default_rng(20240611)


def h(x):
    """binary16 bits of the values x."""
    return np.asarray(x, np.float16).view(np.uint16)


def hv(bits):
    """Exact value (Fraction) of binary16 bits."""
    return F(float(np.uint16(bits).view(np.float16)))


def ulp16(x: float) -> float:
    return float(np.spacing(np.float16(abs(x))))


def test_scale_requant_exact_grid(O):
    # values on a grid that binary16 holds exactly, with both ends present: the codes are
    # the grid indices, the meta is the grid, and the read-back is exact
    for base, step, n in ((0.5, 2.0 ** -10, 128), (0.25, 2.0 ** -11, 128), (3.0, 2.0 ** -6, 77)):
        k = RNG.integers(0, 256, n)
        k[0], k[-1] = 0, 255
        v = (base + k * step).astype(np.float16)
        assert np.array_equal(v.astype(np.float64), base + k * step)   # exact on the grid
        sq, meta = O.scale_requant(v.view(np.uint16), group=128)
        assert np.array_equal(sq, k.astype(np.uint8))
        assert hv(meta[0]) == F(step) and hv(meta[1]) == F(base)
        back = O.scale_dequant(sq, meta, group=128)
        assert np.array_equal(back, v.view(np.uint16))


def test_scale_requant_nearest_code(O):
    # lognormal scales like 1/s of 2-bit groups; ragged last group. Each code is a nearest
    # grid point of {k*step + base, k = 0..255} (exact arithmetic; within 2^-20 step of the
    # best, which admits the binary32 rounding of the quotient), the base is the group's
    # minimum and the step is (max - min)/255 to binary16 precision.
    n, group = 1000, 128
    v = np.exp(RNG.normal(-4.0, 0.6, n)).astype(np.float16)
    sq, meta = O.scale_requant(h(v), group=group)
    assert meta.size == 2 * 8
    for m in range(8):
        blk = v[m * group:(m + 1) * group].astype(np.float64)
        step, base = hv(meta[2 * m]), hv(meta[2 * m + 1])
        assert base == F(blk.min())
        exact_step = (F(blk.max()) - F(blk.min())) / 255
        assert abs(float(step - exact_step)) <= 0.5 * ulp16(float(exact_step)) * (1 + 1e-9)
        codes = sq[m * group:(m + 1) * group]
        for x, c in zip(blk, codes):
            d = [abs(kk * step + base - F(x)) for kk in range(256)]
            best = min(d)
            assert d[int(c)] - best <= step * F(1, 1 << 20)
        assert codes[np.argmin(blk)] == 0


def test_scale_requant_half_step_bound(O):
    n = 4096
    v = np.exp(RNG.normal(-3.0, 1.0, n)).astype(np.float16)
    sq, meta = O.scale_requant(h(v), group=128)
    back = O.scale_dequant(sq, meta, group=128).view(np.float16).astype(np.float64)
    for m in range(n // 128):
        sl = slice(m * 128, (m + 1) * 128)
        step = float(hv(meta[2 * m]))
        err = np.abs(back[sl] - v[sl].astype(np.float64))
        inner = (sq[sl] > 0) & (sq[sl] < 255)
        tol16 = np.array([ulp16(x) for x in back[sl]]) * 0.5
        # half a step on the stored grid, plus the binary16 rounding of the read-back
        assert np.all(err[inner] <= 0.5 * step * (1 + 1e-6) + tol16[inner])
        # the top code clamps at 255: the stored step may be short by half a binary16 ulp
        assert np.all(err <= (0.5 + 255 * 2.0 ** -11) * step + tol16)


def test_scale_requant_groups_are_independent(O):
    n, group = 700, 128
    v = np.exp(RNG.normal(-4.0, 0.5, n)).astype(np.float16)
    sq, meta = O.scale_requant(h(v), group=group)
    w = v.copy()
    w[300] = np.float16(float(v.max()) * 4)          # group 2 only
    sq2, meta2 = O.scale_requant(h(w), group=group)
    other = np.ones(n, bool)
    other[256:384] = False
    assert np.array_equal(sq[other], sq2[other])
    assert np.array_equal(np.delete(meta, [4, 5]), np.delete(meta2, [4, 5]))
    assert not np.array_equal(meta[4:6], meta2[4:6])
    # the short last group (700 = 5*128 + 60) stands alone
    tail_q, tail_meta = O.u8_affine(v[640:].astype(np.float32))
    assert np.array_equal(sq[640:], tail_q) and np.array_equal(meta[10:12], tail_meta)


def test_scale_requant_degenerate(O):
    # a constant group: step 1 (binary16 0x3c00), every code 0, base the value
    sq, meta = O.scale_requant(h(np.full(128, 0.0123)), group=128)
    assert np.all(sq == 0) and meta[0] == 0x3c00 and meta[1] == h(0.0123)
    # group 1: each scale is its own grid
    v = np.exp(RNG.normal(-4, 1, 9)).astype(np.float16)
    sq, meta = O.scale_requant(h(v), group=1)
    assert np.all(sq == 0) and np.array_equal(meta[1::2], h(v)) and np.all(meta[0::2] == 0x3c00)
    assert np.array_equal(O.scale_dequant(sq, meta, group=1), h(v))
    # one value, and none
    sq, meta = O.scale_requant(h([0.5]), group=128)
    assert sq.tolist() == [0] and meta[1] == h(0.5)
    sq, meta = O.scale_requant(np.zeros(0, np.uint16), group=128)
    assert sq.size == 0 and meta.size == 0


def test_scale_requant_matches_zero_rule(O):
    # one group over the whole array is the per-tensor rule of the 8-bit zero-point
    v = np.exp(RNG.normal(-4, 0.7, 300)).astype(np.float16)
    sq, meta = O.scale_requant(h(v), group=300)
    zq, zmeta = O.zero_requant(v.astype(np.float32))
    assert np.array_equal(sq, zq) and np.array_equal(meta, zmeta)
