"""Packed layout of the codes: hand-derived fixtures and an independent numpy packer."""
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
RNG = np.random.default_rng(7)


def fixtures():
    out = []
    with open(os.path.join(HERE, "golden", "pack_layout.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            b, codes, packed = (p.strip() for p in line.split("|"))
            out.append((int(b), np.array([int(c) for c in codes.split()], np.uint8),
                        bytes.fromhex(packed.replace(" ", ""))))
    return out


def numpy_pack(codes, nbits):
    codes = codes.astype(np.uint64)
    if nbits == 3:
        n = len(codes)
        nw = (n + 9) // 10
        c = np.zeros(nw * 10, np.uint64)
        c[:n] = codes
        words = (c.reshape(nw, 10) << (3 * np.arange(10, dtype=np.uint64))).sum(1)
        return words.astype("<u4").tobytes()
    bits = ((codes[:, None] >> np.arange(nbits, dtype=np.uint64)) & 1).astype(np.uint8)
    return np.packbits(bits.reshape(-1), bitorder="little").tobytes()


@pytest.mark.parametrize("case", fixtures(), ids=lambda c: f"b{c[0]}-n{len(c[1])}")
def test_golden_layout(O, case):
    nbits, codes, packed = case
    assert O.pack(codes, nbits).tobytes() == packed
    assert np.array_equal(O.unpack(np.frombuffer(packed, np.uint8), len(codes), nbits), codes)


@pytest.mark.parametrize("nbits", [1, 2, 3, 4, 8])
def test_pack_roundtrip_and_independent_packer(O, nbits):
    for n in list(range(0, 41)) + [1000, 1023, 4097]:
        codes = RNG.integers(0, 1 << nbits, n).astype(np.uint8)
        p = O.pack(codes, nbits)
        expect_len = 4 * ((n + 9) // 10) if nbits == 3 else (n * nbits + 7) // 8
        assert p.size == expect_len == O.packed_bytes(n, nbits)
        assert p.tobytes() == numpy_pack(codes, nbits)
        assert np.array_equal(O.unpack(p, n, nbits), codes)
        if nbits == 3 and p.size:
            words = p.view("<u4")
            assert np.all(words >> 30 == 0)
