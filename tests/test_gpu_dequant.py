"""hqq_dequantize on the GPU (through the C ABI) against the oracle, bit-exact: both kernels
(the flat one for aligned buffers, the element-wise one otherwise), every bit width, both zero
storages, both axes. Inputs are seeded codes, scales and zeros (no solve needed).
Needs an MI355X."""
import numpy as np
import pytest
import torch

import synth
from tests.conftest import has_gpu
from tests.gpu_util import u16

pytestmark = pytest.mark.gpu

if has_gpu():
    from calibration_free_weight_amd import hqq

SENT = -12345


@pytest.fixture(scope="module")
def dev():
    if not has_gpu():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def operands(O, rows, cols, nbits, g, zero_bits, seed):
    rng = np.random.default_rng(seed)
    n, n_groups = rows * cols, rows * cols // g
    codes = rng.integers(0, 1 << nbits, n).astype(np.uint8)
    scale = u16(synth.scale_values(n_groups, seed))
    if zero_bits == 16:
        zero = rng.uniform(-1.0, (1 << nbits) + 1.0, n_groups).astype(np.float16).view(np.uint16)
        meta = None
    else:
        zero = rng.integers(0, 256, n_groups).astype(np.uint8)
        meta = np.array([np.float16(0.0633), np.float16(-1.014)]).view(np.uint16)
    return codes, O.pack(codes, nbits), scale, zero, meta


def run(O, dev, rows, cols, nbits, g, zero_bits, axis, offset, seed):
    codes, packed, scale, zero, meta = operands(O, rows, cols, nbits, g, zero_bits, seed)
    if axis == 1:
        ref = O.dequantize(codes, scale, zero, meta, g, zero_bits)
    else:
        ref = O.dequantize_axis0(codes, scale, zero, meta, rows, cols, g, zero_bits)
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(dev)
    n = rows * cols
    buf = torch.full((n + offset + 16,), SENT, dtype=torch.int16, device=dev)
    out = buf[offset:offset + n]
    hqq.hqq_dequantize(t(packed, np.uint8), t(scale, np.int16),
                       t(zero, np.int16 if zero_bits == 16 else np.uint8),
                       None if meta is None else t(meta, np.int16), rows, cols, nbits, g, axis,
                       zero_bits, out)
    torch.cuda.synchronize()
    b = u16(buf)
    assert np.array_equal(b[offset:offset + n], ref)
    assert np.all(b[:offset] == np.uint16(SENT & 0xFFFF)) and \
        np.all(b[offset + n:] == np.uint16(SENT & 0xFFFF)), "written outside W_out"


@pytest.mark.parametrize("offset", [0, 1])         # 16-byte aligned output, or not
@pytest.mark.parametrize("zero_bits", [16, 8])
@pytest.mark.parametrize("nbits", [1, 2, 3, 4, 8])
def test_dequantize_axis1(O, dev, nbits, zero_bits, offset):
    for g, rows, cols in ((16, 37, 48), (64, 5, 640), (256, 9, 512), (128, 1, 128)):
        print(f"dequantize axis 1 nbits={nbits} g={g} zb={zero_bits} {rows}x{cols} "
              f"offset={offset}", flush=True)
        run(O, dev, rows, cols, nbits, g, zero_bits, 1, offset, 100 * nbits + g + rows)


@pytest.mark.parametrize("zero_bits", [16, 8])
@pytest.mark.parametrize("nbits", [1, 2, 3, 4, 8])
def test_dequantize_axis0(O, dev, nbits, zero_bits):
    # cols a multiple of 8 takes the flat kernel, 131 the element-wise one
    for g, rows, cols, offset in ((16, 48, 136, 0), (64, 128, 131, 0), (32, 64, 200, 1),
                                  (128, 256, 8, 0)):
        print(f"dequantize axis 0 nbits={nbits} g={g} zb={zero_bits} {rows}x{cols} "
              f"offset={offset}", flush=True)
        run(O, dev, rows, cols, nbits, g, zero_bits, 0, offset, 300 * nbits + g + cols)


def test_dequantize_large(O, dev):
    # a 33.6 M-element weight: 4100 blocks, each thread four units a grid apart
    rows, cols, nbits, g = 2050, 16384, 4, 64
    print(f"dequantize {rows}x{cols}", flush=True)
    run(O, dev, rows, cols, nbits, g, 8, 1, 0, 7)
