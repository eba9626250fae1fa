"""hqq_quantize_noalloc (static scratch, no workspace argument) gives what hqq_quantize gives,
on two calls in a row, the second with a smaller input (needs an MI355X)."""
import numpy as np
import pytest
import torch

from tests.conftest import has_gpu
from tests.gpu_util import u16, u8, weights

pytestmark = pytest.mark.gpu

if has_gpu():
    from calibration_free_weight_amd import hqq


@pytest.fixture(scope="module")
def dev():
    if not has_gpu():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def outputs_equal(a, b, label):
    for k in ("packed", "scale", "zero", "zero_meta", "passes"):
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), f"{label}: {k} differs"


@pytest.mark.parametrize("nbits,g,zero_bits", [(4, 64, 16), (4, 128, 8), (3, 64, 8),
                                               (2, 16, 8)])
def test_noalloc_matches_workspace_call(O, dev, nbits, g, zero_bits):
    # two calls in a row on the shared scratch, the second smaller: each must match the
    # workspace entry point bit for bit (and the first the oracle)
    for i, (rows, cols) in enumerate(((1024, 4096), (96, 2 * g * 5))):
        label = f"noalloc call {i} {rows}x{cols} b{nbits} g{g} z{zero_bits}"
        print(label, flush=True)
        W = weights(rows, cols, 4200 + i + nbits + g, dev)
        ref = hqq.quantize(W, nbits, g, zero_bits=zero_bits, passes=True)
        out = hqq.alloc_outputs(rows, cols, nbits, g, zero_bits, dev, passes=True)
        hqq.hqq_quantize_noalloc(W, nbits, g, 1, 0.7, 1.0, 1.01, 20, 1, zero_bits,
                                 out["packed"], out["scale"], out["zero"], out["zero_meta"],
                                 out["passes"])
        torch.cuda.synchronize()
        outputs_equal(out, ref, label)
        if i == 0:
            r = O.quantize(u16(W), g, nbits, zero_bits=zero_bits)
            assert np.array_equal(u8(out["packed"])[:r["packed"].size], r["packed"]), label


def test_noalloc_axis0_and_limit(dev):
    W = weights(256, 512, 77, dev)
    ref = hqq.quantize(W, 4, 64, axis=0, zero_bits=8, passes=True)
    out = hqq.alloc_outputs(256, 512, 4, 64, 8, dev, passes=True)
    hqq.hqq_quantize_noalloc(W, 4, 64, 0, 0.7, 1.0, 1.01, 20, 1, 8, out["packed"], out["scale"],
                             out["zero"], out["zero_meta"], out["passes"])
    torch.cuda.synchronize()
    outputs_equal(out, ref, "noalloc axis 0")
    # an axis-0 tensor whose transposed copy exceeds the 64 MiB scratch is refused up front
    Wb = torch.empty(8192, 8192, dtype=torch.float16, device=dev)
    big = hqq.alloc_outputs(8192, 8192, 4, 64, 16, dev)
    with pytest.raises(hqq.HQQError) as e:
        hqq.hqq_quantize_noalloc(Wb, 4, 64, 0, 0.7, 1.0, 1.01, 20, 1, 16, big["packed"],
                                 big["scale"], big["zero"], None, None)
    assert e.value.status == hqq.HQQ_ERR_WORKSPACE
