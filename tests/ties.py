"""Seeded inputs whose reconstruction lands on a binary16 rounding tie (test inputs only).

A value that is rounded to binary32 and then to binary16 can differ from the same exact value
rounded to binary16 once: when the binary32 result is exactly halfway between two binary16
values while the exact result lies on the odd side of that midpoint. The generators below
search seeded random operands for such cases, so that a path which merges the two roundings
fails. Candidates are found with numpy binary64/binary32 arithmetic (products and sums that
are exact in binary64 are formed there, then rounded once); expected values in the tests come
from the oracle."""
import numpy as np

_BATCH = 1 << 20
_MAX_BATCHES = 64


def _f16_tie(t64):
    """t64 (float64 holding binary32 values): True where t64 is a binary16 midpoint."""
    h = t64.astype(np.float16)                               # round to nearest even
    other = np.where(h.astype(np.float64) <= t64, np.nextafter(h, np.float16(np.inf)),
                     np.nextafter(h, np.float16(-np.inf)))
    return (np.abs(t64 - h.astype(np.float64)) == np.abs(other.astype(np.float64) - t64)) & \
        np.isfinite(other.astype(np.float64))


def _collect(count, seed, draw):
    rng = np.random.default_rng(seed)
    parts = []
    for _ in range(_MAX_BATCHES):
        parts.append(draw(rng))
        if sum(p[0].size for p in parts) >= count:
            return tuple(np.concatenate([p[i] for p in parts])[:count] for i in range(len(parts[0])))
    raise RuntimeError("too few tie cases found")


def dequant_ties(count, seed, step, base, nbits=4):
    """(q, zq, s16) for a tensor with 8-bit zeros on the grid {step, base} (binary16): codes,
    zero codes and binary16 scales with binary32((q - binary32(zq*step + base)) * s) a
    binary16 tie that single rounding would resolve the other way."""
    st, bs = np.float64(np.float16(step)), np.float64(np.float16(base))

    def draw(rng):
        q = rng.integers(0, 1 << nbits, _BATCH)
        zq = rng.integers(0, 256, _BATCH)
        s = np.exp(rng.uniform(np.log(1e-3), np.log(0.2), _BATCH)).astype(np.float16)
        zf = (zq * st + bs).astype(np.float32)               # exact in binary64, one rounding
        d = np.float32(q) - zf
        v = (d * s.astype(np.float32)).astype(np.float64)     # binary32 product
        exact = d.astype(np.float64) * s.astype(np.float64)   # 24 x 11 bits: exact in binary64
        keep = _f16_tie(v) & (exact.astype(np.float16) != v.astype(np.float16)) & (v != 0)
        return q[keep].astype(np.uint8), zq[keep].astype(np.uint8), s[keep]
    return _collect(count, seed, draw)


def scale_dequant_ties(count, seed):
    """(q, step16, base16): 8-bit scale codes and run meta with binary32(q*step + base) a
    binary16 tie that single rounding would resolve the other way (a small step next to a
    large base, so that the sum is inexact in binary32)."""
    def draw(rng):
        q = rng.integers(0, 256, _BATCH)
        step = np.exp(rng.uniform(np.log(6.2e-5), np.log(4e-4), _BATCH)).astype(np.float16)
        base = np.exp(rng.uniform(np.log(0.5), np.log(4.0), _BATCH)).astype(np.float16)
        exact = q * step.astype(np.float64) + base.astype(np.float64)   # exact in binary64
        v = exact.astype(np.float32).astype(np.float64)                 # one binary32 rounding
        keep = _f16_tie(v) & (exact.astype(np.float16) != v.astype(np.float16))
        return q[keep].astype(np.uint8), step[keep], base[keep]
    return _collect(count, seed, draw)
