"""8-bit scales on the GPU (through the C ABI) against the oracle: bit-exact codes, meta and
read-back, from single values to the scale count of a 2-bit g16 Llama-2-7B-shaped stack.
Needs an MI355X."""
import numpy as np
import pytest
import torch

import synth
from tests.conftest import has_gpu
from tests.gpu_util import u16, u8, weights

pytestmark = pytest.mark.gpu

if has_gpu():
    from calibration_free_weight_amd import hqq

RNG = np.random.default_rng(777)
SENT = 0xAB
SIZES = [1, 7, 8, 9, 100, 127, 128, 129, 1000, 4101, 3 * 65536 + 11]
STACK_SCALES = 6_476_005_376 // 16         # 2-bit g16 Llama-2-7B-shaped stack


@pytest.fixture(scope="module")
def dev():
    if not has_gpu():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def gpu_requant(v16: torch.Tensor, group: int):
    """Requant on the device into sentinel-filled buffers; returns (codes, meta) on the host
    and checks that nothing was written past the outputs."""
    n = v16.numel()
    n_runs = (n + group - 1) // group
    sq = torch.full((n + 64,), SENT, dtype=torch.uint8, device=v16.device)
    meta = torch.full((2 * n_runs + 8,), SENT, dtype=torch.int16, device=v16.device)
    hqq.hqq_requant_scales(v16, n, group, sq, meta)
    torch.cuda.synchronize()
    q, m = u8(sq), u16(meta)
    assert np.all(q[n:] == SENT), "scale_q written past n"
    assert np.all(m[2 * n_runs:] == np.uint16(SENT)), "scale_meta written past its runs"
    return q[:n], m[:2 * n_runs]


@pytest.mark.parametrize("group", [8, 16, 64, 128, 512])
def test_scale_requant_matches_oracle(O, dev, group):
    for n in SIZES:
        print(f"scale requant group={group} n={n}", flush=True)
        v = synth.scale_values(n, 1000 + n, device=dev)
        q, m = gpu_requant(v, group)
        rq, rm = O.scale_requant(u16(v), group=group)
        assert np.array_equal(q, rq), f"codes n={n}"
        assert np.array_equal(m, rm), f"meta n={n}"


def test_scale_requant_special_runs(O, dev):
    group = 128
    runs = [
        np.full(group, 0.0123),                                   # constant: step 1
        0.5 + RNG.integers(0, 256, group) * 2.0 ** -10,           # exact grid
        np.repeat([0.01, 0.02], group // 2),                      # two values
        np.exp(RNG.normal(-17, 0.5, group)),                      # binary16 subnormals
        np.exp(RNG.normal(9, 1.0, group)).clip(max=65000),        # large scales
        np.r_[np.full(group - 1, 0.01), 60000.0],                 # one outlier: all else code 0
        # exact ties: grid 0.5 + k/1024 (both ends present) with values at half steps, so
        # (v - base)/step is exactly k + 1/2 and must round to even
        np.r_[0.5, 0.5 + 255 / 1024, 0.5 + (RNG.integers(0, 255, group - 2) + 0.5) / 1024],
    ]
    v = np.concatenate(runs).astype(np.float16)
    vt = torch.from_numpy(v.view(np.int16)).to(dev)
    q, m = gpu_requant(vt, group)
    rq, rm = O.scale_requant(v.view(np.uint16), group=group)
    assert np.array_equal(q, rq) and np.array_equal(m, rm)
    ties = q[-group + 2:].astype(np.int64)
    assert np.all(ties % 2 == 0), "half-step ties round to even"


@pytest.mark.parametrize("group", [8, 128, 512])
def test_scale_dequant_matches_oracle(O, dev, group):
    for n in SIZES:
        print(f"scale dequant group={group} n={n}", flush=True)
        v = u16(synth.scale_values(n, 2000 + n, device=dev))
        rq, rm = O.scale_requant(v, group=group)
        ref = O.scale_dequant(rq, rm, group=group)
        qt = torch.from_numpy(rq).to(dev)
        mt = torch.from_numpy(rm.view(np.int16)).to(dev)
        out = torch.full((n + 64,), SENT, dtype=torch.int16, device=dev)
        hqq.hqq_dequantize_scales(qt, mt, n, group, out)
        torch.cuda.synchronize()
        o = u16(out)
        assert np.array_equal(o[:n], ref), f"n={n}"
        assert np.all(o[n:] == np.uint16(SENT)), "scale_out written past n"


def test_scale_requant_stack_size_sampled(O, dev):
    # the 2-bit g16 7B-shaped stack's scale count plus a ragged run, in one launch; sampled
    # runs (first, last and 3000 random ones) against the oracle run by run
    group = 128
    n = STACK_SCALES + 77
    print(f"scale requant stack size n={n}", flush=True)
    v = synth.scale_values(n, 31337, device=dev)
    sq, meta = hqq.requant_scales(v, group)
    torch.cuda.synchronize()
    n_runs = (n + group - 1) // group
    pick = np.unique(np.r_[0, n_runs - 1, RNG.integers(0, n_runs, 3000)])
    idx = torch.from_numpy(pick).to(dev)
    vv = v[: (n_runs - 1) * group].view(n_runs - 1, group)
    tail = u16(v[(n_runs - 1) * group:])
    full = pick[pick < n_runs - 1]
    vs = u16(vv[idx[: full.size]]).reshape(-1, group)
    qs = u8(sq[: (n_runs - 1) * group].view(n_runs - 1, group)[idx[: full.size]]).reshape(-1, group)
    ms = u16(meta.view(n_runs, 2)[idx]).reshape(-1, 2)
    for r, m in enumerate(full):
        rq, rm = O.scale_requant(vs[r], group=group)
        assert np.array_equal(qs[r], rq) and np.array_equal(ms[r], rm), f"run {m}"
    rq, rm = O.scale_requant(tail, group=group)
    assert np.array_equal(u8(sq[(n_runs - 1) * group:]), rq) and np.array_equal(ms[-1], rm)
    del v, sq, meta


def test_g16_s_variant_end_to_end(O, dev):
    # 2-bit g16 with 8-bit zero (per tensor) and 8-bit scales (runs of 128): solve, requant the
    # scales, read them back, reconstruct; each step bit-exact with the oracle's own chain
    rows, cols, nbits, g = 64, 2048 + 16 * 7, 2, 16
    W = weights(rows, cols, 4242, dev)
    out = hqq.quantize(W, nbits, g, zero_bits=8)
    sq, smeta = hqq.requant_scales(out["scale"], 128)
    n_groups = rows * cols // g
    back = torch.empty(n_groups, dtype=torch.float16, device=dev)
    hqq.hqq_dequantize_scales(sq, smeta, n_groups, 128, back)
    Wr = torch.empty_like(W)
    hqq.hqq_dequantize(out["packed"], back, out["zero"], out["zero_meta"], rows, cols, nbits, g,
                       1, 8, Wr)
    torch.cuda.synchronize()
    ref = O.quantize(u16(W), g, nbits, zero_bits=8)
    assert np.array_equal(u16(out["scale"]), ref["scale"])
    rq, rm = O.scale_requant(ref["scale"], group=128)
    assert np.array_equal(u8(sq), rq) and np.array_equal(u16(smeta), rm)
    rback = O.scale_dequant(rq, rm, group=128)
    assert np.array_equal(u16(back), rback)
    rW = O.dequantize(ref["codes"], rback, ref["zero"], ref["zero_meta"], g, 8)
    assert np.array_equal(u16(Wr), rW)


def test_scale_dequant_ties_bit_exact(O, dev):
    # runs whose binary32 fma(q, step, base) is a binary16 tie that a merged (single) rounding
    # would resolve the other way: the read-back must round to binary32 first, as the oracle
    from tests import ties
    q, st, bs = ties.scale_dequant_ties(64, 22)
    group = 8
    meta = np.stack([st, bs], axis=1).reshape(-1).view(np.uint16)
    codes = np.repeat(q, group)
    ref = O.scale_dequant(codes, meta, group=group)
    out = torch.empty(codes.size, dtype=torch.int16, device=dev)
    hqq.hqq_dequantize_scales(torch.from_numpy(codes).to(dev),
                              torch.from_numpy(meta.view(np.int16)).to(dev), codes.size, group, out)
    torch.cuda.synchronize()
    assert np.array_equal(u16(out), ref)
