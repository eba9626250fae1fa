"""Empty inputs on every entry point that launches work: each returns HQQ_OK and launches
nothing that reads its (possibly null) buffers (needs an MI355X)."""
import pytest
import torch

from tests.conftest import has_gpu

pytestmark = pytest.mark.gpu

if has_gpu():
    from calibration_free_weight_amd import hqq


@pytest.fixture(scope="module")
def dev():
    if not has_gpu():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.mark.parametrize("shape,axis", [((5, 0), 1), ((0, 64), 1), ((0, 128), 0), ((64, 0), 0)])
@pytest.mark.parametrize("zero_bits", [16, 8])
def test_empty_tensor_quantize(dev, shape, axis, zero_bits):
    print(f"empty quantize {shape} axis {axis} z{zero_bits}", flush=True)
    W = torch.empty(shape, dtype=torch.float16, device=dev)
    out = hqq.quantize(W, 4, 64, axis=axis, zero_bits=zero_bits, passes=True)
    torch.cuda.synchronize()
    assert out["scale"].numel() == 0 and out["zero"].numel() == 0
    o2 = hqq.alloc_outputs(shape[0], shape[1], 4, 64, zero_bits, dev, passes=True)
    hqq.hqq_quantize_noalloc(W, 4, 64, axis, 0.7, 1.0, 1.01, 20, 1, zero_bits, o2["packed"],
                             o2["scale"], o2["zero"], o2["zero_meta"], o2["passes"])
    torch.cuda.synchronize()


def test_empty_calls_of_the_other_entry_points(dev):
    print("empty dequantize / pack / unpack / scales / gemm_f16", flush=True)
    for rows, cols in ((0, 64), (3, 0)):
        W = torch.empty(rows, cols, dtype=torch.float16, device=dev)
        hqq.hqq_dequantize(None, None, None, None, rows, cols, 4, 64, 1, 16, W)
    hqq.hqq_pack(None, 0, 3, None)
    hqq.hqq_unpack(None, 0, 4, None)
    hqq.hqq_requant_scales(None, 0, 128, None, None)
    hqq.hqq_dequantize_scales(None, None, 0, 128, None)
    X = torch.empty(0, 64, dtype=torch.float16, device=dev)
    Wr = torch.zeros(16, 64, dtype=torch.float16, device=dev)
    Y = torch.empty(0, 16, dtype=torch.float16, device=dev)
    hqq.hqq_gemm_f16(X, Wr, 16, 64, Y)
    Xm = torch.zeros(4, 64, dtype=torch.float16, device=dev)
    hqq.hqq_gemm_f16(Xm, Wr, 0, 64, torch.empty(4, 0, dtype=torch.float16, device=dev))
    torch.cuda.synchronize()
