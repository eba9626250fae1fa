"""Axis-0 grouping (groups down columns) on the GPU, through the C ABI, against the oracle:
bit-exact codes, packed bytes, scales, zeros, meta and evaluation counts. Needs an MI355X."""
import numpy as np
import pytest
import torch

import synth
from tests.conftest import has_gpu
from tests.gpu_util import u16, u8, weights

pytestmark = pytest.mark.gpu

if has_gpu():
    from calibration_free_weight_amd import hqq

RNG = np.random.default_rng(31)


@pytest.fixture(scope="module")
def dev():
    if not has_gpu():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def check_axis0(O, W, out, nbits, g, zero_bits, label):
    rows, cols = W.shape
    ref = O.quantize_axis0(u16(W), rows, cols, g, nbits, zero_bits=zero_bits)
    n = rows * cols
    packed = u8(out["packed"])[:ref["packed"].size]
    codes = O.unpack(packed, n, nbits)
    nd = int((codes != ref["codes"]).sum())
    assert nd == 0, f"{label}: {nd} codes differ"
    assert np.array_equal(packed, ref["packed"]), f"{label}: packed bytes"
    assert np.array_equal(u16(out["scale"]), ref["scale"]), f"{label}: scale"
    zero = u16(out["zero"]) if zero_bits == 16 else u8(out["zero"])
    assert np.array_equal(zero, ref["zero"]), f"{label}: {(zero != ref['zero']).sum()} zeros"
    if zero_bits == 8:
        assert np.array_equal(u16(out["zero_meta"]), ref["zero_meta"]), f"{label}: meta"
    if out.get("passes") is not None:
        ok = ref["shrink_active"] == 0
        got = u8(out["passes"])
        assert np.array_equal(got[ok], ref["evals_needed"][ok]), f"{label}: pass counts"
    return ref


@pytest.mark.parametrize("zero_bits", [16, 8])
@pytest.mark.parametrize("g", [16, 64, 128, 256])
@pytest.mark.parametrize("nbits", [1, 2, 3, 4, 8])
def test_axis0_matches_oracle(O, dev, nbits, g, zero_bits):
    rows, cols = 3 * g, 131                 # ragged against the 64 x 64 transpose tiles
    label = f"axis0 nbits={nbits} g={g} zero_bits={zero_bits} {rows}x{cols}"
    print(label, flush=True)
    W = weights(rows, cols, 7000 + 10 * nbits + g, dev)
    out = hqq.quantize(W, nbits, g, axis=0, zero_bits=zero_bits, passes=True)
    torch.cuda.synchronize()
    check_axis0(O, W, out, nbits, g, zero_bits, label)


@pytest.mark.parametrize("nbits,g,zero_bits", [(4, 64, 16), (2, 16, 8), (3, 128, 8)])
def test_axis0_dequantize_matches_oracle(O, dev, nbits, g, zero_bits):
    rows, cols = 4 * g, 77
    w16 = synth.half_bits(synth.student_t_weights(rows, cols, 91 + g)).reshape(-1)
    ref = O.quantize_axis0(w16, rows, cols, g, nbits, zero_bits=zero_bits)
    back = O.dequantize_axis0(ref["codes"], ref["scale"], ref["zero"], ref["zero_meta"], rows,
                              cols, g, zero_bits)
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(dev)
    packed = t(ref["packed"], np.uint8)
    scale = t(ref["scale"], np.int16)
    zero = t(ref["zero"], np.int16 if zero_bits == 16 else np.uint8)
    meta = None if zero_bits == 16 else t(ref["zero_meta"], np.int16)
    Wr = torch.empty(rows, cols, dtype=torch.float16, device=dev)
    hqq.hqq_dequantize(packed, scale, zero, meta, rows, cols, nbits, g, 0, zero_bits, Wr)
    torch.cuda.synchronize()
    assert np.array_equal(u16(Wr), back)


def test_axis0_and_axis1_in_one_batch(O, dev):
    # one launch sequence over tensors of both axes, bit widths and zero storage
    specs = [(0, 4, 64, 16, 192, 200), (1, 4, 64, 16, 70, 256), (0, 2, 16, 8, 64, 96),
             (1, 3, 32, 8, 33, 320), (0, 3, 32, 8, 96, 50), (0, 8, 128, 16, 256, 9)]
    jobs, outs, Ws = [], [], []
    for i, (axis, nbits, g, zb, rows, cols) in enumerate(specs):
        W = weights(rows, cols, 8100 + i, dev)
        o = hqq.alloc_outputs(rows, cols, nbits, g, zb, dev, passes=True)
        jobs.append(hqq.make_job(W, nbits, g, axis, 0.7, 1.0, 1.01, 20, 1, zb, o["packed"],
                                 o["scale"], o["zero"], o["zero_meta"], o["passes"]))
        Ws.append(W)
        outs.append(o)
    ws = hqq.alloc_workspace(jobs, dev)
    hqq.hqq_quantize_batch(jobs, ws)
    torch.cuda.synchronize()
    for (axis, nbits, g, zb, rows, cols), W, o in zip(specs, Ws, outs):
        label = f"batch axis={axis} nbits={nbits} g={g} zb={zb}"
        if axis == 0:
            check_axis0(O, W, o, nbits, g, zb, label)
        else:
            ref = O.quantize(u16(W), g, nbits, zero_bits=zb)
            assert np.array_equal(u8(o["packed"])[:ref["packed"].size], ref["packed"]), label
            assert np.array_equal(u16(o["scale"]), ref["scale"]), label
            zero = u16(o["zero"]) if zb == 16 else u8(o["zero"])
            assert np.array_equal(zero, ref["zero"]), label
            if zb == 8:
                assert np.array_equal(u16(o["zero_meta"]), ref["zero_meta"]), label
            ok = ref["shrink_active"] == 0
            assert np.array_equal(u8(o["passes"])[ok], ref["evals_needed"][ok]), label


def test_axis0_stack_sampled(O, dev):
    # the Llama-2-7B-shaped stack (224 tensors, 4-bit g128, binary16 zeros) with groups down
    # columns, in one batch; 40 sampled column runs per tensor against the oracle
    specs = synth.workload(2)
    jobs, keep = [], []
    for s in specs:
        W = synth.student_t_weights(s.rows, s.cols, s.seed(2), device=dev)
        o = hqq.alloc_outputs(s.rows, s.cols, 4, 128, 16, dev)
        jobs.append(hqq.make_job(W, 4, 128, 0, 0.7, 1.0, 1.01, 20, 1, 16, o["packed"], o["scale"],
                                 o["zero"], o["zero_meta"]))
        keep.append((W, o))
    ws = hqq.alloc_workspace(jobs, dev)
    print(f"axis-0 stack: {len(jobs)} tensors, workspace {ws.numel() / 2**30:.1f} GiB", flush=True)
    hqq.hqq_quantize_batch(jobs, ws)
    torch.cuda.synchronize()
    del ws
    for t, (s, (W, o)) in enumerate(zip(specs, keep)):
        nb = s.rows // 128
        b = RNG.integers(0, nb, 40)
        j = RNG.integers(0, s.cols, 40)
        rows_idx = (b[:, None] * 128 + np.arange(128)[None, :])          # [40, 128]
        ri = torch.from_numpy(rows_idx).to(dev)
        ci = torch.from_numpy(np.repeat(j[:, None], 128, axis=1)).to(dev)
        runs = u16(W[ri, ci]).reshape(40, 128)
        ref = O.solve_groups(runs.reshape(-1), 128, 4)
        pos = rows_idx.astype(np.int64) * s.cols + j[:, None]           # 4-bit codes, LSB first
        byt = u8(o["packed"][torch.from_numpy(pos // 2).to(dev)]).reshape(pos.shape)
        got_codes = (byt >> (4 * (pos % 2))) & 15
        assert np.array_equal(got_codes.reshape(-1), ref["codes"]), f"tensor {t} codes"
        gi = b * s.cols + j
        assert np.array_equal(u16(o["scale"])[gi], ref["scale"]), f"tensor {t} scale"
        assert np.array_equal(u16(o["zero"])[gi], O.zero_to_half(ref["zero_f32"])), \
            f"tensor {t} zero"


@pytest.mark.parametrize("nbits", [1, 2, 4, 8])
@pytest.mark.parametrize("cols", [256, 136, 104, 131])
def test_axis0_code_write_back_paths(O, dev, nbits, cols):
    # the packed codes go back to the tensor's order by 32-bit words (rows*nbits and
    # cols*nbits multiples of 32), by bytes (multiples of 8), or unpack + transpose + pack
    rows, g = 64, 16
    label = f"axis0 write-back nbits={nbits} cols={cols}"
    print(label, flush=True)
    W = weights(rows, cols, 9100 + nbits + cols, dev)
    out = hqq.quantize(W, nbits, g, axis=0, zero_bits=16, passes=True)
    torch.cuda.synchronize()
    check_axis0(O, W, out, nbits, g, 16, label)
