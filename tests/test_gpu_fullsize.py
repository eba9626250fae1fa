"""Whole-tensor parity at the workloads' full sizes (needs an MI355X).

Every distinct (shape, bit width, group size) of the model-shaped stacks is quantized as a
whole tensor and compared element by element with the oracle: packed bytes, scales, the
binary32 zeros, the 8-bit zeros and their step/base, and the evaluation counts. The oracle
is the single-threaded C oracle run over disjoint ranges of groups in several processes.
The last test quantizes the whole Llama-2-7B-shaped stack (224 tensors, 6.48e9 weights)
in one batched call and compares every tensor the same way.
"""
import time

import pytest
import torch

import synth
from tests.conftest import has_gpu
from tests.gpu_util import compare_whole

pytestmark = pytest.mark.gpu

if has_gpu():
    from calibration_free_weight_amd import hqq


@pytest.fixture(scope="module")
def dev():
    if not has_gpu():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def pool():
    from oracle.pool import OraclePool
    with OraclePool() as P:
        yield P


# (workload, projection index, rows, cols, nbits, g): block 0 of each stack, one tensor per
# distinct shape and setting; every stack stores 8-bit zeros.
SHAPES = [
    (2, 0, 4096, 4096, 4, 128), (2, 4, 11008, 4096, 4, 128), (2, 6, 4096, 11008, 4, 128),
    (3, 0, 4096, 4096, 2, 16), (3, 4, 11008, 4096, 2, 16), (3, 6, 4096, 11008, 2, 16),
    (4, 0, 5120, 5120, 4, 64), (4, 4, 13824, 5120, 2, 32), (4, 6, 5120, 13824, 2, 32),
    (5, 0, 8192, 8192, 3, 64), (5, 1, 1024, 8192, 3, 64), (5, 4, 28672, 8192, 3, 64),
    (5, 6, 8192, 28672, 3, 64),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("workload,proj,rows,cols,nbits,g", SHAPES)
def test_whole_tensor(O, pool, dev, progress, workload, proj, rows, cols, nbits, g):
    label = f"workload {workload} {synth.PROJ[proj]} {rows}x{cols} {nbits}-bit g{g}"
    progress(f"whole tensor: {label}")
    W = synth.student_t_weights(rows, cols, synth.seed_for(workload, 0, proj), device=dev)
    out = hqq.quantize(W, nbits, g, zero_bits=8, passes=True)
    torch.cuda.synchronize()
    ng = rows * cols // g
    z32 = out["workspace"][:4 * ng].view(torch.float32)   # the one job's zeros come first
    t = time.perf_counter()
    ref = compare_whole(O, pool, W, out, nbits, g, 8, zero32=z32, label=label)
    progress(f"  equal; oracle on {pool.procs} processes {time.perf_counter() - t:.1f} s, "
             f"{int(ref['shrink_active'].sum())} groups with a live shrink")


@pytest.mark.timeout(900)
def test_whole_llama2_7b_stack(O, pool, dev, progress):
    """All 224 tensors of the 7B-shaped stack (4-bit g128, 8-bit zeros) in one batch."""
    specs = synth.workload(2)
    Ws, outs, jobs = [], [], []
    for s in specs:
        W = synth.student_t_weights(s.rows, s.cols, s.seed(2), device=dev)
        o = hqq.alloc_outputs(s.rows, s.cols, s.nbits, s.group_size, s.zero_bits, dev,
                              passes=True)
        jobs.append(hqq.make_job(W, s.nbits, s.group_size, 1, 0.7, 1.0, 1.01, 20, 1,
                                 s.zero_bits, o["packed"], o["scale"], o["zero"],
                                 o["zero_meta"], o["passes"]))
        Ws.append(W)
        outs.append(o)
    ws = hqq.alloc_workspace(jobs, dev)
    hqq.hqq_quantize_batch(jobs, ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, (s, W, o) in enumerate(zip(specs, Ws, outs)):
        if s.proj == 0:
            progress(f"7B stack: block {s.block} ({time.perf_counter() - t0:.0f} s)")
        compare_whole(O, pool, W, o, s.nbits, s.group_size, s.zero_bits, label=s.name)
    progress(f"7B stack: 224 tensors equal; oracle wall time {time.perf_counter() - t0:.1f} s "
             f"on {pool.procs} processes")
