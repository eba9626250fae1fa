"""The quantized linear layer Y = X . W_r^T on the GPU (through the C ABI) against the
oracle. Needs an MI355X.

Tolerance, from the arithmetic: W_r is the same binary16 reconstruction on both sides and each
product of two binary16 values is exact in binary32, so the GPU result differs from the
binary64 oracle only by the binary32 summation (at most K+1 roundings of partial sums, each
within 2^-24 of the running magnitude: (K+1)·2^-24·sum|x||w|) and the final rounding to
binary16 (half an ulp: 2^-11·|y|, or 2^-25 below the normal range)."""
import numpy as np
import pytest
import torch

import synth
from tests.conftest import has_gpu
from tests.gpu_util import u16

pytestmark = pytest.mark.gpu

if has_gpu():
    from calibration_free_weight_amd import hqq

RNG = np.random.default_rng(4040)


@pytest.fixture(scope="module")
def dev():
    if not has_gpu():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def qweight(O, n, k, nbits, g, zero_bits, seed):
    """Oracle-quantized weight [n, k] (inputs of the GEMM come from the oracle, not the GPU)."""
    w16 = synth.half_bits(synth.student_t_weights(n, k, seed)).reshape(-1)
    r = O.quantize(w16, g, nbits, zero_bits=zero_bits)
    return r


def to_dev(a, dt, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(dev)


def run_gemm(r, x16, m, n, k, nbits, g, zero_bits, dev, workspace=False):
    X = to_dev(x16, np.int16, dev).view(m, k)
    packed = to_dev(r["packed"], np.uint8, dev)
    scale = to_dev(r["scale"], np.int16, dev)
    zero = to_dev(r["zero"], np.int16 if zero_bits == 16 else np.uint8, dev)
    meta = None if zero_bits == 16 else to_dev(r["zero_meta"], np.int16, dev)
    Y = torch.full((m, n), float("nan"), dtype=torch.float16, device=dev)
    ws = None
    if workspace:
        wb = hqq.hqq_gemm_workspace_bytes(m, n, k)
        ws = torch.full((max(wb, 1),), 0x7E, dtype=torch.uint8, device=dev)
    hqq.hqq_gemm(X, packed, scale, zero, meta, n, k, nbits, g, zero_bits, Y, workspace=ws)
    torch.cuda.synchronize()
    return u16(Y).view(np.float16).astype(np.float64).reshape(m, n)


def check(O, r, x16, y, m, n, k, g, zero_bits, label):
    ref = O.gemm(x16, r["codes"], r["scale"], r["zero"], r["zero_meta"], n, k, g, zero_bits)
    w = O.dequantize(r["codes"], r["scale"], r["zero"], r["zero_meta"], g, zero_bits)
    w = np.abs(w.view(np.float16).astype(np.float64).reshape(n, k))
    x = np.abs(x16.view(np.float16).astype(np.float64).reshape(m, k))
    tol = (k + 1) * 2.0 ** -24 * (x @ w.T) + np.maximum(2.0 ** -11 * np.abs(ref), 2.0 ** -25)
    err = np.abs(y - ref)
    assert not np.isnan(y).any(), f"{label}: unwritten outputs"
    assert np.all(err <= tol * (1 + 1e-9)), f"{label}: max err/tol {np.max(err / tol):.3f}"
    return ref


@pytest.mark.parametrize("nbits,g,zero_bits", [(4, 128, 8), (4, 16, 16), (2, 32, 8),
                                               (3, 64, 16), (8, 16, 8), (1, 64, 16),
                                               (1, 16, 8)])
@pytest.mark.parametrize("m", [1, 3, 8, 9, 64, 100])
def test_gemm_matches_oracle(O, dev, nbits, g, zero_bits, m):
    n, k = 200, 1024 + 16 * (g == 16)        # ragged against the 128-wide tiles; K % 64 = 16
    r = qweight(O, n, k, nbits, g, zero_bits, 10 * nbits + g)
    x16 = synth.half_bits(synth.student_t_weights(m, k, 3 + m)).reshape(-1)
    x16 = (x16.view(np.float16).astype(np.float32) * 40).astype(np.float16).view(np.uint16)
    for ws in (False, True) if m > 64 else (False,):
        label = f"gemm m={m} n={n} k={k} nbits={nbits} g={g} zero_bits={zero_bits} ws={ws}"
        print(label, flush=True)
        y = run_gemm(r, x16, m, n, k, nbits, g, zero_bits, dev, workspace=ws)
        check(O, r, x16, y, m, n, k, g, zero_bits, label)


@pytest.mark.parametrize("nbits,g,zero_bits", [(4, 16, 8), (8, 32, 16), (2, 16, 16)])
def test_gemm_decode_ragged(O, dev, nbits, g, zero_bits):
    # the decode kernels on ragged shapes: odd N (a wave's second row missing), one row,
    # K below one chunk of 32 codes per lane, between chunks, and past one 2048-code sweep
    # (with g = 16, K % 32 == 16: a lane's last chunk ends half past the row), past two
    # sweeps (M = 1: three chunks per lane in flight) and past four (two rounds of three, the
    # second partly past the row); packed buffers offset by 4 bytes (still word-aligned) and
    # by 1 byte (the fallback)
    for m in (1, 2, 5, 8):
        for n, k in ((1, g), (3, 3 * g), (201, 2048 + g), (7, 4096 + g), (5, 8192 + 3 * g)):
            r = qweight(O, n, k, nbits, g, zero_bits, 31 * n + k + nbits)
            x16 = synth.half_bits(synth.student_t_weights(m, k, 7 + m + k)).reshape(-1)
            for shift in (0, 4, 1):
                label = f"decode m={m} n={n} k={k} nbits={nbits} g={g} zb={zero_bits} shift={shift}"
                print(label, flush=True)
                X = to_dev(x16, np.int16, dev).view(m, k)
                pk = torch.zeros(r["packed"].size + 16, dtype=torch.uint8, device=dev)
                pk[shift:shift + r["packed"].size] = to_dev(r["packed"], np.uint8, dev)
                scale = to_dev(r["scale"], np.int16, dev)
                zero = to_dev(r["zero"], np.int16 if zero_bits == 16 else np.uint8, dev)
                meta = None if zero_bits == 16 else to_dev(r["zero_meta"], np.int16, dev)
                Y = torch.full((m, n), float("nan"), dtype=torch.float16, device=dev)
                hqq.hqq_gemm(X, pk[shift:], scale, zero, meta, n, k, nbits, g, zero_bits, Y)
                torch.cuda.synchronize()
                y = u16(Y).view(np.float16).astype(np.float64).reshape(m, n)
                check(O, r, x16, y, m, n, k, g, zero_bits, label)


@pytest.mark.parametrize("nbits,g,zero_bits", [(4, 16, 8), (3, 32, 16), (8, 16, 16), (1, 64, 8),
                                               (4, 64, 16), (8, 64, 8), (4, 32, 8)])
def test_gemm_skinny_ragged(O, dev, nbits, g, zero_bits):
    # the matrix-core skinny kernel (8 < M <= 64): one to four 16-row M tiles, N below, at and
    # past one 16-row block, K of one 32-wide step (most of the block's waves idle), a few
    # steps, and a half step at the end
    for m in (9, 17, 33, 48, 64):
        for n, k in ((15, g), (16, 3 * g), (17, 64 + g), (200, 4096 + g)):
            label = f"skinny m={m} n={n} k={k} nbits={nbits} g={g} zb={zero_bits}"
            print(label, flush=True)
            r = qweight(O, n, k, nbits, g, zero_bits, 17 * n + k + nbits)
            x16 = synth.half_bits(synth.student_t_weights(m, k, 5 + m + k)).reshape(-1)
            x16 = (x16.view(np.float16).astype(np.float32) * 40).astype(np.float16).view(np.uint16)
            y = run_gemm(r, x16, m, n, k, nbits, g, zero_bits, dev)
            check(O, r, x16, y, m, n, k, g, zero_bits, label)


@pytest.mark.parametrize("nbits,g,zero_bits", [(4, 16, 8), (2, 32, 16)])
def test_gemm_unaligned_packed_fallback(O, dev, nbits, g, zero_bits):
    # a packed buffer on an odd address: the word-reading kernels step aside and the original
    # ones (per-row decode for M <= 8, LDS-staged tiles above) take every M
    n, k = 131, 1024 + g
    r = qweight(O, n, k, nbits, g, zero_bits, 41 + nbits)
    for m, with_ws in ((3, False), (9, False), (100, False), (100, True)):
        # with a workspace, M = 100 would reconstruct once; an unaligned packed buffer must
        # keep it off that path's word loads
        label = f"unaligned m={m} ws={with_ws} nbits={nbits} g={g} zb={zero_bits}"
        print(label, flush=True)
        x16 = synth.half_bits(synth.student_t_weights(m, k, 9 + m)).reshape(-1)
        X = to_dev(x16, np.int16, dev).view(m, k)
        pk = torch.zeros(r["packed"].size + 16, dtype=torch.uint8, device=dev)
        pk[1:1 + r["packed"].size] = to_dev(r["packed"], np.uint8, dev)
        Y = torch.full((m, n), float("nan"), dtype=torch.float16, device=dev)
        wb = hqq.hqq_gemm_workspace_bytes(m, n, k)
        ws = torch.empty(wb, dtype=torch.uint8, device=dev) if with_ws and wb else None
        assert not with_ws or ws is not None
        hqq.hqq_gemm(X, pk[1:], to_dev(r["scale"], np.int16, dev),
                     to_dev(r["zero"], np.int16 if zero_bits == 16 else np.uint8, dev),
                     None if zero_bits == 16 else to_dev(r["zero_meta"], np.int16, dev),
                     n, k, nbits, g, zero_bits, Y, workspace=ws)
        torch.cuda.synchronize()
        y = u16(Y).view(np.float16).astype(np.float64).reshape(m, n)
        check(O, r, x16, y, m, n, k, g, zero_bits, label)


@pytest.mark.parametrize("m,n,k", [(65, 128, 16), (130, 129, 48), (257, 300, 2064),
                                   (200, 1, 32), (512, 256, 4096), (520, 8200, 272),
                                   (1000, 8200, 80)])
def test_gemm_workspace_path_shapes(O, dev, m, n, k):
    # the reconstruct-once path: ragged M and N against the 64 x 128 and 128 x 128 tiles (the
    # last shape has enough blocks for the taller ones), K below one 64-step and with a 16- or
    # 48-wide tail, a single output column, grids not a multiple of the 8 XCDs; without the
    # workspace the same inputs run through the streaming kernels (64-row slices above 64)
    nbits, g, zero_bits = 4, 16, 8
    r = qweight(O, n, k, nbits, g, zero_bits, 5 + m + n + k)
    x16 = synth.half_bits(synth.student_t_weights(m, k, 17 + m)).reshape(-1)
    x16 = (x16.view(np.float16).astype(np.float32) * 40).astype(np.float16).view(np.uint16)
    for ws in (True, False):
        label = f"gemm shape m={m} n={n} k={k} ws={ws}"
        print(label, flush=True)
        y = run_gemm(r, x16, m, n, k, nbits, g, zero_bits, dev, workspace=ws)
        check(O, r, x16, y, m, n, k, g, zero_bits, label)


def test_gemm_layer_shape_sampled(O, dev):
    # a 7B MLP layer shape (N = 11008, K = 4096, 4-bit g128) at decode (M = 1) and prefill
    # (M = 512) sizes. The GPU quantizes and multiplies the whole layer; the oracle quantizes
    # the sampled rows from the same weights (binary16 zeros: rows are independent) and
    # computes the sampled outputs.
    n, k, nbits, g = 11008, 4096, 4, 128
    W = synth.student_t_weights(n, k, 77, device=dev)
    out = hqq.quantize(W, nbits, g, zero_bits=16)
    torch.cuda.synchronize()
    rows = np.unique(RNG.integers(0, n, 48))
    ridx = torch.from_numpy(rows).to(dev)
    ref_w = O.quantize(u16(W[ridx]).reshape(-1), g, nbits, zero_bits=16)
    w = O.dequantize(ref_w["codes"], ref_w["scale"], ref_w["zero"], None, g, 16)
    w = np.abs(w.view(np.float16).astype(np.float64).reshape(rows.size, k))
    for m, use_ws in ((1, False), (512, False), (512, True)):
        print(f"gemm layer shape m={m} workspace={use_ws}", flush=True)
        X = synth.student_t_weights(m, k, 900 + m, device=dev).mul_(40)
        Y = torch.full((m, n), float("nan"), dtype=torch.float16, device=dev)
        ws = None
        if use_ws:
            ws = torch.empty(hqq.hqq_gemm_workspace_bytes(m, n, k), dtype=torch.uint8,
                             device=dev)
        hqq.hqq_gemm(X, out["packed"], out["scale"], out["zero"], None, n, k, nbits, g, 16, Y,
                     workspace=ws)
        torch.cuda.synchronize()
        ms = np.unique(RNG.integers(0, m, min(m, 16)))
        midx = torch.from_numpy(ms).to(dev)
        x16 = u16(X[midx]).reshape(-1)
        ref = O.gemm(x16, ref_w["codes"], ref_w["scale"], ref_w["zero"], None, rows.size, k, g,
                     16)
        y = u16(Y[midx][:, ridx]).view(np.float16).astype(np.float64).reshape(ms.size, rows.size)
        xa = np.abs(x16.view(np.float16).astype(np.float64).reshape(ms.size, k))
        tol = (k + 1) * 2.0 ** -24 * (xa @ w.T) + np.maximum(2.0 ** -11 * np.abs(ref), 2.0 ** -25)
        assert np.all(np.abs(y - ref) <= tol * (1 + 1e-9)), f"m={m}"
        assert not torch.isnan(Y).any(), f"m={m}: unwritten outputs"


def test_reconstruction_ties_bit_exact(O, dev):
    # weights whose binary32 reconstruction is a binary16 tie that a merged (single) rounding
    # would resolve the other way (8-bit zeros: the zero is a full binary32 value). With X the
    # identity, Y = W_r^T exactly on every path: hqq_dequantize, the decode kernel (M <= 8),
    # the fused matrix-core kernel and the reconstruct-once path (M = 128)
    from tests import ties
    step, base, g, k = 0.0633, -1.014, 16, 128
    q, zq, s = ties.dequant_ties(32 * (k // g), 21, step, base)
    n = q.size // (k // g)
    meta = np.array([np.float16(step), np.float16(base)]).view(np.uint16)
    codes = np.repeat(q, g)
    ref = O.dequantize(codes, s.view(np.uint16), zq, meta, g, 8).view(np.float16).reshape(n, k)
    packed = to_dev(O.pack(codes, 4), np.uint8, dev)
    scale, zero, zmeta = to_dev(s, np.int16, dev), to_dev(zq, np.uint8, dev), to_dev(meta, np.int16, dev)
    Wr = torch.empty(n, k, dtype=torch.float16, device=dev)
    hqq.hqq_dequantize(packed, scale, zero, zmeta, n, k, 4, g, 1, 8, Wr)
    torch.cuda.synchronize()
    assert np.array_equal(Wr.cpu().numpy(), ref), "hqq_dequantize"
    eye = torch.eye(k, dtype=torch.float16, device=dev)
    for m, use_ws in ((1, False), (8, False), (128, False), (128, True)):
        print(f"ties m={m} workspace={use_ws}", flush=True)
        Y = torch.full((m, n), float("nan"), dtype=torch.float16, device=dev)
        ws = torch.empty(max(hqq.hqq_gemm_workspace_bytes(m, n, k), 1), dtype=torch.uint8,
                         device=dev) if use_ws else None
        hqq.hqq_gemm(eye[:m].contiguous(), packed, scale, zero, zmeta, n, k, 4, g, 8, Y,
                     workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(Y.cpu().numpy(), ref[:, :m].T), f"m={m} workspace={use_ws}"


def run_f16(x16, w16, m, n, k, dev):
    X = to_dev(x16, np.int16, dev).view(m, k)
    W = to_dev(w16, np.int16, dev).view(n, k)
    Y = torch.full((m, n), float("nan"), dtype=torch.float16, device=dev)
    hqq.hqq_gemm_f16(X, W, n, k, Y)
    torch.cuda.synchronize()
    return u16(Y).view(np.float16).astype(np.float64).reshape(m, n)


@pytest.mark.parametrize("m,n,k", [(1, 1, 8), (3, 15, 24), (65, 200, 1032), (129, 130, 8),
                                   (300, 257, 4104)])
def test_gemm_f16_matches_binary64_product(dev, m, n, k):
    # hqq_gemm_f16 on a plain binary16 weight: M = 1, one output column, K of one 8-wide
    # chunk and with 8- and 24-wide tails past the 64-wide steps, ragged M and N against the
    # tiles; the reference is the binary64 product (a library matmul), the tolerance the
    # binary32 summation plus the final rounding, as for hqq_gemm
    x16 = synth.half_bits(synth.student_t_weights(m, k, 31 + m)).reshape(-1)
    x16 = (x16.view(np.float16).astype(np.float32) * 40).astype(np.float16).view(np.uint16)
    w16 = synth.half_bits(synth.student_t_weights(n, k, 37 + n)).reshape(-1)
    print(f"gemm_f16 m={m} n={n} k={k}", flush=True)
    y = run_f16(x16, w16, m, n, k, dev)
    x = x16.view(np.float16).astype(np.float64).reshape(m, k)
    w = w16.view(np.float16).astype(np.float64).reshape(n, k)
    ref = x @ w.T
    tol = (k + 1) * 2.0 ** -24 * (np.abs(x) @ np.abs(w).T) + np.maximum(2.0 ** -11 * np.abs(ref), 2.0 ** -25)
    assert not np.isnan(y).any(), "unwritten outputs"
    assert np.all(np.abs(y - ref) <= tol * (1 + 1e-9)), f"max err/tol {np.max(np.abs(y - ref) / tol):.3f}"


@pytest.mark.parametrize("m,n,k", [(130, 129, 48), (520, 8200, 272)])
def test_gemm_f16_equals_workspace_path(O, dev, m, n, k):
    # the two-step layer (the oracle's W_r, then hqq_gemm_f16) and hqq_gemm's reconstruct-once
    # path run one kernel on the same W_r, so Y is identical
    nbits, g, zero_bits = 4, 16, 8
    r = qweight(O, n, k, nbits, g, zero_bits, 41 + m + n + k)
    x16 = synth.half_bits(synth.student_t_weights(m, k, 43 + m)).reshape(-1)
    wr = O.dequantize(r["codes"], r["scale"], r["zero"], r["zero_meta"], g, zero_bits)
    print(f"gemm_f16 vs workspace m={m} n={n} k={k}", flush=True)
    y2 = run_f16(x16, np.ascontiguousarray(wr).view(np.uint16).reshape(-1), m, n, k, dev)
    y1 = run_gemm(r, x16, m, n, k, nbits, g, zero_bits, dev, workspace=True)
    assert not np.isnan(y2).any()
    assert np.array_equal(y1, y2)


def _random_weight(n, k, nbits, g, zero_bits, dev, gen, offset=0):
    """A quantized weight with random codes, scales and zeros (every byte pattern is a valid
    code stream): enough to compare two ways of multiplying it. `offset` shifts the packed
    buffer off its allocation's alignment."""
    nbytes = hqq.hqq_packed_bytes(n * k, nbits)
    buf = torch.randint(0, 256, (nbytes + 16,), dtype=torch.uint8, device=dev, generator=gen)
    ng = n * k // g
    scale = (torch.rand(ng, device=dev, generator=gen) * 0.02 + 0.001).to(torch.float16)
    if zero_bits == 16:
        zero = (torch.rand(ng, device=dev, generator=gen) * 15).to(torch.float16)
        meta = None
    else:
        zero = torch.randint(0, 256, (ng,), dtype=torch.uint8, device=dev, generator=gen)
        meta = torch.tensor([0.0625, -1.5], dtype=torch.float16, device=dev)
    return dict(packed=buf[offset:offset + nbytes], scale=scale, zero=zero, zero_meta=meta, N=n,
                nbits=nbits, group_size=g, zero_bits=zero_bits)


@pytest.mark.parametrize("m,workspace", [(1, False), (2, False), (5, False), (16, False),
                                         (33, False), (64, False), (100, False), (100, True)])
def test_gemm_multi_equals_single_calls(dev, m, workspace):
    """hqq_gemm_multi writes, for every weight, exactly what hqq_gemm writes for it alone:
    weights of several bit widths, group sizes and zero storages, ragged N, more weights than
    one shared launch takes, and one packed buffer off its alignment (its own launch)."""
    k = 1024
    gen = torch.Generator(device=dev)
    gen.manual_seed(77 + m)
    specs = [(64, 4, 128, 8), (200, 4, 64, 16), (48, 2, 16, 8), (17, 8, 32, 16), (96, 3, 64, 8),
             (100, 1, 128, 16)] + [(16 * (i + 1) + i, 4, 128, 8) for i in range(9)]
    ws_ = [_random_weight(n, k, b, g, zb, dev, gen) for n, b, g, zb in specs]
    ws_.append(_random_weight(40, k, 4, 64, 16, dev, gen, offset=1))
    X = (torch.randn(m, k, device=dev, generator=gen) * 0.5).to(torch.float16)
    work = None
    if workspace:
        wb = max(hqq.hqq_gemm_workspace_bytes(m, w["N"], k) for w in ws_)
        work = torch.empty(wb, dtype=torch.uint8, device=dev)
    for w in ws_:
        w["Y"] = torch.full((m, w["N"]), float("nan"), dtype=torch.float16, device=dev)
    print(f"multi m={m} workspace={workspace}: {len(ws_)} weights", flush=True)
    hqq.hqq_gemm_multi(X, ws_, workspace=work)
    torch.cuda.synchronize()
    for i, w in enumerate(ws_):
        single = torch.full_like(w["Y"], float("nan"))
        hqq.hqq_gemm(X, w["packed"], w["scale"], w["zero"], w["zero_meta"], w["N"], k, w["nbits"],
                     w["group_size"], w["zero_bits"], single, workspace=work)
        torch.cuda.synchronize()
        assert torch.equal(w["Y"].view(torch.int16), single.view(torch.int16)), \
            f"weight {i} {specs[i] if i < len(specs) else 'unaligned'}"


def test_gemm_empty_k_writes_zeros(dev):
    # K = 0 is an empty sum: Y = 0 on every path (decode, skinny, sliced and workspace M), and
    # neither X nor the weight buffers are read, so they may be null
    nan = float("nan")
    for m in (1, 5, 64, 100):
        for nbits, zb in ((4, 8), (3, 16), (2, 16)):
            label = f"empty K m={m} nbits={nbits} zb={zb}"
            print(label, flush=True)
            X = torch.empty((m, 0), dtype=torch.float16, device=dev)
            Y = torch.full((m, 37), nan, dtype=torch.float16, device=dev)
            ws = torch.zeros(256, dtype=torch.uint8, device=dev) if m > 64 else None
            hqq.hqq_gemm(X, None, None, None, None, 37, 0, nbits, 64, zb, Y, workspace=ws)
            torch.cuda.synchronize()
            assert bool((Y == 0).all()), label
    X = torch.empty((7, 0), dtype=torch.float16, device=dev)
    Ys = [torch.full((7, n), nan, dtype=torch.float16, device=dev) for n in (16, 33, 5)]
    hqq.hqq_gemm_multi(X, [dict(packed=None, scale=None, zero=None, zero_meta=None, N=Y.shape[1],
                                nbits=nb, group_size=128, zero_bits=16, Y=Y)
                           for Y, nb in zip(Ys, (4, 4, 8))])
    torch.cuda.synchronize()
    assert all(bool((Y == 0).all()) for Y in Ys)
