"""Host-streamed quantization on the GPU (weights in pinned host memory, copied chunk by chunk
into a staging buffer while the previous chunk is solved) against the oracle. Needs an
MI355X."""
import numpy as np
import pytest
import torch

from tests.conftest import has_gpu
from tests.gpu_util import u16, u8, weights
from tests.test_gpu_axis0 import check_axis0

pytestmark = pytest.mark.gpu

if has_gpu():
    from calibration_free_weight_amd import hqq


@pytest.fixture(scope="module")
def dev():
    if not has_gpu():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


SPECS = [(1, 4, 64, 16, 96, 512), (0, 2, 16, 8, 64, 200), (1, 3, 32, 8, 40, 320),
         (1, 8, 128, 16, 33, 256), (0, 4, 128, 8, 256, 64), (1, 1, 16, 16, 70, 96),
         (1, 4, 256, 8, 20, 512), (0, 3, 64, 16, 128, 40)]


def _host_jobs(dev, seed0):
    host, outs, jobs = [], [], []
    for i, (axis, nbits, g, zb, rows, cols) in enumerate(SPECS):
        Wd = weights(rows, cols, seed0 + i, dev)
        Wh = torch.empty(rows, cols, dtype=torch.float16, pin_memory=True)
        Wh.copy_(Wd.cpu())
        o = hqq.alloc_outputs(rows, cols, nbits, g, zb, dev, passes=True)
        jobs.append(hqq.make_job(Wh, nbits, g, axis, 0.7, 1.0, 1.01, 20, 1, zb, o["packed"],
                                 o["scale"], o["zero"], o["zero_meta"], o["passes"]))
        host.append((Wh, Wd))
        outs.append(o)
    return host, outs, jobs


@pytest.mark.parametrize("copy_stream", [False, True])
def test_streamed_matches_oracle(O, dev, copy_stream):
    host, outs, jobs = _host_jobs(dev, 600)
    largest = max(2 * r * c for (_, _, _, _, r, c) in SPECS)
    staging_bytes = 2 * ((largest + 255) // 256 * 256)      # one tensor per half at most
    staging = torch.empty(staging_bytes, dtype=torch.uint8, device=dev)
    n_ws = hqq.hqq_streamed_workspace_bytes(jobs, staging_bytes)
    ws = torch.empty(max(n_ws, 256), dtype=torch.uint8, device=dev)
    cs = torch.cuda.Stream() if copy_stream else None
    print(f"streamed: {len(jobs)} tensors, staging {staging_bytes} B, copy stream {copy_stream}",
          flush=True)
    hqq.hqq_quantize_streamed(jobs, staging, ws, None,
                              None if cs is None else cs.cuda_stream)
    torch.cuda.synchronize()
    for (axis, nbits, g, zb, rows, cols), (Wh, Wd), o in zip(SPECS, host, outs):
        label = f"streamed axis={axis} nbits={nbits} g={g} zb={zb}"
        if axis == 0:
            check_axis0(O, Wd, o, nbits, g, zb, label)
        else:
            ref = O.quantize(u16(Wd), g, nbits, zero_bits=zb)
            assert np.array_equal(u8(o["packed"])[:ref["packed"].size], ref["packed"]), label
            assert np.array_equal(u16(o["scale"]), ref["scale"]), label
            zero = u16(o["zero"]) if zb == 16 else u8(o["zero"])
            assert np.array_equal(zero, ref["zero"]), label
            ok = ref["shrink_active"] == 0
            assert np.array_equal(u8(o["passes"])[ok], ref["evals_needed"][ok]), label


def test_streamed_equals_in_memory_batch(dev):
    # several tensors per chunk, and chunks reusing both halves more than once
    host, outs, jobs = _host_jobs(dev, 700)
    staging_bytes = 2 * 160 * 1024
    staging = torch.empty(staging_bytes, dtype=torch.uint8, device=dev)
    ws = torch.empty(max(hqq.hqq_streamed_workspace_bytes(jobs, staging_bytes), 256),
                     dtype=torch.uint8, device=dev)
    cs = torch.cuda.Stream()
    hqq.hqq_quantize_streamed(jobs, staging, ws, None, cs.cuda_stream)
    dev_jobs, dev_outs = [], []
    for (axis, nbits, g, zb, rows, cols), (Wh, Wd) in zip(SPECS, host):
        o = hqq.alloc_outputs(rows, cols, nbits, g, zb, dev, passes=True)
        dev_jobs.append(hqq.make_job(Wd, nbits, g, axis, 0.7, 1.0, 1.01, 20, 1, zb, o["packed"],
                                     o["scale"], o["zero"], o["zero_meta"], o["passes"]))
        dev_outs.append(o)
    hqq.hqq_quantize_batch(dev_jobs, hqq.alloc_workspace(dev_jobs, dev))
    torch.cuda.synchronize()
    for a, b in zip(outs, dev_outs):
        for k in ("packed", "scale", "zero", "zero_meta", "passes"):
            if a[k] is not None:
                assert torch.equal(a[k], b[k]), k


def test_consecutive_streamed_calls_share_staging(O, dev):
    """Two calls in a row on one staging buffer with a separate copy stream: the second
    call's first copies must wait for the first call's last solves, which still read the
    staging halves."""
    staging_bytes = 2 * 160 * 1024
    staging = torch.empty(staging_bytes, dtype=torch.uint8, device=dev)
    cs = torch.cuda.Stream()
    calls = [_host_jobs(dev, 900), _host_jobs(dev, 950)]
    ws = torch.empty(max(max(hqq.hqq_streamed_workspace_bytes(j, staging_bytes)
                             for _, _, j in calls), 256), dtype=torch.uint8, device=dev)
    for host, outs, jobs in calls:
        hqq.hqq_quantize_streamed(jobs, staging, ws, None, cs.cuda_stream)
    torch.cuda.synchronize()
    for n, (host, outs, jobs) in enumerate(calls):
        for (axis, nbits, g, zb, rows, cols), (Wh, Wd), o in zip(SPECS, host, outs):
            label = f"call {n} axis={axis} nbits={nbits} g={g} zb={zb}"
            if axis == 0:
                check_axis0(O, Wd, o, nbits, g, zb, label)
                continue
            ref = O.quantize(u16(Wd), g, nbits, zero_bits=zb)
            assert np.array_equal(u8(o["packed"])[:ref["packed"].size], ref["packed"]), label
            assert np.array_equal(u16(o["scale"]), ref["scale"]), label
            zero = u16(o["zero"]) if zb == 16 else u8(o["zero"])
            assert np.array_equal(zero, ref["zero"]), label


def test_streamed_rejects_a_tensor_larger_than_half(dev):
    host, outs, jobs = _host_jobs(dev, 800)
    staging = torch.empty(2 * 4096, dtype=torch.uint8, device=dev)
    with pytest.raises(hqq.HQQError) as e:
        hqq.hqq_quantize_streamed(jobs, staging, None)
    assert e.value.status == hqq.HQQ_ERR_WORKSPACE
