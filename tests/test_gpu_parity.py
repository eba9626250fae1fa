"""Parity of the HIP path (through the C ABI) with the CPU oracle. Needs an MI355X."""
import numpy as np
import pytest
import torch

from tests.conftest import has_gpu
import synth
from tests.gpu_util import compare, u16, u8, weights

pytestmark = pytest.mark.gpu

if has_gpu():
    from calibration_free_weight_amd import hqq

RNG = np.random.default_rng(2024)


@pytest.fixture(scope="module")
def dev():
    if not has_gpu():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run(W, nbits, g, zero_bits=16, passes=True, check=True, **params):
    out = hqq.quantize(W, nbits, g, zero_bits=zero_bits, passes=passes, **params)
    torch.cuda.synchronize()
    if check and out["workspace"] is not None:
        hqq.hqq_batch_check([out["job"]], out["workspace"])   # no group left unwritten
    return out


# ---------------------------------------------------------------------------------------
# pack / unpack: bit-exact
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("nbits", [1, 2, 3, 4, 8])
def test_pack_unpack_bitexact(O, dev, nbits):
    for n in [1, 9, 10, 11, 15, 16, 17, 31, 33, 1000, 4097, 65539]:
        print(f"pack nbits={nbits} n={n}", flush=True)
        codes = RNG.integers(0, 1 << nbits, n).astype(np.uint8)
        ct = torch.from_numpy(codes).to(dev)
        nb = hqq.hqq_packed_bytes(n, nbits)
        packed = torch.full((nb + 16,), 0xAB, dtype=torch.uint8, device=dev)
        hqq.hqq_pack(ct, n, nbits, packed)
        back = torch.zeros(n + 8, dtype=torch.uint8, device=dev)
        hqq.hqq_unpack(packed, n, nbits, back)
        torch.cuda.synchronize()
        p = u8(packed)
        assert np.array_equal(p[:nb], O.pack(codes, nbits))
        assert np.all(p[nb:] == 0xAB), "pack wrote past the packed size"
        b = u8(back)
        assert np.array_equal(b[:n], codes) and np.all(b[n:] == 0)


# ---------------------------------------------------------------------------------------
# quantize: every bit width x group size x zero storage, several blocks and a ragged tail
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("zero_bits", [16, 8])
@pytest.mark.parametrize("g", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("nbits", [1, 2, 3, 4, 8])
def test_quantize_matches_oracle(O, dev, nbits, g, zero_bits):
    rows, cols = 67, g * 20          # 1340 groups: several blocks, last one partial
    print(f"quantize {rows}x{cols} nbits={nbits} g={g} zero={zero_bits}", flush=True)
    W = weights(rows, cols, 100 * nbits + g + zero_bits, dev)
    out = run(W, nbits, g, zero_bits)
    compare(O, W, out, nbits, g, zero_bits, label=f"b{nbits} g{g} z{zero_bits}")


@pytest.mark.parametrize("layout", [1, 2, 3], ids=["wide", "narrow", "lockstep"])
@pytest.mark.parametrize("nbits", [1, 2, 3, 4, 8])
def test_both_pass_layouts(O, dev, nbits, layout):
    """The solver's kernels (persistent with one lane per group or several lanes per group;
    lockstep, chosen for small batches) give identical results: forced here for every bit
    width and group size, on boundary groups that exercise the exact path, with 8-bit zeros
    and with a live shrink."""
    try:
        hqq.hqq_debug_solver(pass_layout=layout)
        for g in (16, 32, 64, 128, 256):
            print(f"layout {layout} nbits={nbits} g={g}", flush=True)
            W = half_grid_groups(40, g * 24, g, nbits, 300 + nbits + g, 0.3).to(dev)
            for zero_bits in (16, 8):
                out = run(W, nbits, g, zero_bits)
                compare(O, W, out, nbits, g, zero_bits, label=f"layout {layout} b{nbits} g{g}")
            out = run(W, nbits, g, 16, beta=1e4)
            compare(O, W, out, nbits, g, 16, exact=False, params={"beta": 1e4},
                    label=f"layout {layout} shrink b{nbits} g{g}")
    finally:
        hqq.hqq_debug_solver()


@pytest.mark.parametrize("nbits,g", [(4, 64), (2, 16), (3, 64)])
def test_no_early_stop_and_rtn(O, dev, nbits, g):
    W = weights(32, 2048, 5 + nbits, dev)
    for params in ({"iters": 0}, {"early_stop": False}, {"iters": 5}, {"iters": 254}):
        print(f"params {params}", flush=True)
        out = run(W, nbits, g, **params)
        compare(O, W, out, nbits, g, 16, params=params, label=str(params))


def test_edge_inputs(O, dev):
    cases = {
        "constant": torch.full((8, 256), 0.375, dtype=torch.float16),
        "zeros": torch.zeros(8, 256, dtype=torch.float16),
        "two_valued": torch.where(torch.rand(8, 256, generator=torch.Generator().manual_seed(1)) < 0.5,
                                  torch.tensor(-0.0625), torch.tensor(0.1875)).half(),
        "subnormal_only": (torch.randint(-1023, 1024, (8, 256),
                                         generator=torch.Generator().manual_seed(2)).float()
                           * 2.0 ** -24).half(),
        "huge": (torch.randn(8, 256, generator=torch.Generator().manual_seed(3)) * 8000).half(),
        "one_group": torch.randn(1, 16, generator=torch.Generator().manual_seed(4)).half(),
    }
    for name, Wc in cases.items():
        for nbits in (2, 4):
            print(f"edge {name} nbits={nbits}", flush=True)
            W = Wc.to(dev)
            g = 16
            out = run(W, nbits, g)
            compare(O, W, out, nbits, g, 16, label=name)


def magnitude_band_weights(rows, cols, seed, amax):
    """Synthetic weights scaled so that the largest magnitude is amax, with 1 % of the
    entries replaced by binary16 subnormals of either sign: every tile then takes the same
    branch of the solver's binary64 sum of x*s (chains of 4, 2 or 1 exact pair sums below
    1/8, 1/4 and 1/2; products one by one from 1/2 up)."""
    gen = torch.Generator().manual_seed(seed)
    W = synth.student_t_weights(rows, cols, seed).float()
    W = (W * (amax / W.abs().max())).half()
    n = W.numel()
    idx = torch.randperm(n, generator=gen)[: n // 100]
    k = torch.randint(1, 1024, (idx.numel(),), generator=gen)
    sign = torch.where(torch.rand(idx.numel(), generator=gen) < 0.5, 0x8000, 0)
    flat = W.reshape(-1).view(torch.int16)
    flat[idx] = (k | sign).to(torch.int16)
    assert float(W.abs().max()) <= amax * (1 + 2.0 ** -10)
    return W


@pytest.mark.parametrize("amax", [3.0, 0.45, 0.2, 0.1, 2.0 ** -14])
@pytest.mark.parametrize("layout", [1, 3], ids=["persistent", "lockstep"])
def test_weight_magnitude_bands(O, dev, layout, amax):
    """Each branch of the binary64 sum of x*s at the min-max start (by the tile's largest
    magnitude), in both solver kernels, bit-exact against the oracle."""
    try:
        hqq.hqq_debug_solver(pass_layout=layout)
        for g in (16, 64, 128):
            for zero_bits in (16, 8):
                print(f"layout {layout} amax {amax} g={g} zero={zero_bits}", flush=True)
                W = magnitude_band_weights(32, g * 24, 700 + g, amax).to(dev)
                out = run(W, 4, g, zero_bits)
                compare(O, W, out, 4, g, zero_bits, label=f"layout {layout} amax {amax} g{g}")
    finally:
        hqq.hqq_debug_solver()


def half_grid_groups(rows, cols, g, nbits, seed, frac=1.0):
    """Groups whose first evaluation lands exactly on rounding boundaries: each group holds
    its min 0, its max qmax/16 and otherwise values (k + 1/2)/16, so s = 16, z0 = 0 and
    u = k + 1/2 (ties to even). A fraction `frac` of the groups is built this way, the rest
    are ordinary weights. Every such group needs the exact path at its first evaluation."""
    qmax = (1 << nbits) - 1
    gen = torch.Generator().manual_seed(seed)
    ng = rows * cols // g
    W = synth.student_t_weights(rows, cols, seed).reshape(ng, g).clone()
    k = torch.randint(0, qmax, (ng, g), generator=gen).float()
    grid = ((k + 0.5) / 16.0).half()
    grid[:, 0] = 0.0
    grid[:, 1] = qmax / 16.0
    perm = torch.argsort(torch.rand(ng, g, generator=gen), dim=1)
    grid = torch.gather(grid, 1, perm)
    pick = torch.rand(ng, generator=gen) < frac
    W[pick] = grid[pick]
    return W.reshape(rows, cols)


@pytest.mark.parametrize("frac", [1.0, 0.5])
@pytest.mark.parametrize("nbits,g", [(4, 128), (4, 64), (2, 16), (3, 64), (8, 256)])
def test_boundary_groups_take_exact_path(O, dev, nbits, g, frac):
    """Every first evaluation of these groups is a tie of codes: the batch of exact-path
    groups fills the staging slots, so groups are exchanged between lanes and slots."""
    rows, cols = 48, g * 32
    print(f"boundary groups nbits={nbits} g={g} frac={frac}", flush=True)
    W = half_grid_groups(rows, cols, g, nbits, 11 + nbits + g, frac).to(dev)
    for zero_bits in (16, 8):
        out = run(W, nbits, g, zero_bits)
        compare(O, W, out, nbits, g, zero_bits, label=f"grid b{nbits} g{g} z{zero_bits}")


def test_minimal_staging_pool(O, dev):
    """The stress build of the library (a pool of one batch plus four slots) must give the
    same results: free slots are then scarce, so holders swap their group with a ready one
    in place (groups up to 64) or through the spare slot (larger groups), paths the normal
    pool size rarely needs."""
    import os
    from calibration_free_weight_amd import build as hbuild
    assert os.path.exists(hbuild.STRESS_LIB), "build the library (stress build included) first"
    saved = hqq.LIB_PATH, hqq._L
    hqq.LIB_PATH, hqq._L = hbuild.STRESS_LIB, None
    try:
        cases = [(4, 128, 1.0), (4, 128, 0.5), (2, 16, 1.0), (2, 32, 0.5), (3, 32, 1.0),
                 (4, 64, 0.0), (3, 64, 0.3), (8, 256, 0.0)]
        for layout in (1, 2):
            hqq.hqq_debug_solver(pass_layout=layout)
            for nbits, g, frac in cases:
                print(f"stress pool layout={layout} nbits={nbits} g={g} frac={frac}", flush=True)
                W = half_grid_groups(48, g * 32, g, nbits, 5 + nbits + g, frac).to(dev)
                for zero_bits in (16, 8):
                    out = run(W, nbits, g, zero_bits)
                    compare(O, W, out, nbits, g, zero_bits, label=f"stress b{nbits} g{g}")
    finally:
        hqq.hqq_debug_solver()
        hqq.LIB_PATH, hqq._L = saved


def test_step_budget_exhaustion_is_reported(O, dev):
    """A solver wave that runs out of its step budget flags the batch: the host sets a tiny
    budget (every wave still exits normally), and the check reports the incomplete outputs;
    the next solve on the same workspace clears the flag."""
    W = weights(64, 2048, 55, dev)
    try:
        for layout in (1, 3):                     # persistent and lockstep solvers
            hqq.hqq_debug_solver(step_budget=2, pass_layout=layout)
            for zero_bits in (16, 8):
                print(f"tiny step budget, layout={layout} zero_bits={zero_bits}", flush=True)
                out = run(W, 4, 64, zero_bits, check=False)
                with pytest.raises(hqq.HQQError) as e:
                    hqq.hqq_batch_check([out["job"]], out["workspace"])
                assert e.value.status == hqq.HQQ_ERR_DEVICE
                assert "step budget" in str(e.value)
    finally:
        hqq.hqq_debug_solver()
    job, ws = out["job"], out["workspace"]
    hqq.hqq_quantize_batch([job], ws)                 # same outputs and workspace, default budget
    hqq.hqq_batch_check([job], ws)
    compare(O, W, out, 4, 64, 8, label="after the flag")


def test_empty_tensor(dev):
    W = torch.empty(0, 64, dtype=torch.float16, device=dev)
    out = run(W, 4, 64)
    assert out["scale"].numel() == 0


@pytest.mark.parametrize("params", [{"beta": 1e4}, {"p": 1.0}, {"p": 0.5, "beta": 50.0}])
def test_active_shrink_within_tolerance(O, dev, params):
    """With a large beta the shrink moves residuals (the pow branch runs): parity is the
    tolerance bar, not bit equality (binary64 pow differs between libraries in the last bit)."""
    W = weights(64, 1024, 77, dev)
    print(f"shrink {params}", flush=True)
    out = run(W, 4, 64, **params)
    ref = compare(O, W, out, 4, 64, 16, exact=False, params=params, label=str(params))
    if params.get("beta", 1.0) > 100:
        assert ref["shrink_active"].mean() > 0.5


# ---------------------------------------------------------------------------------------
# full-size tensors
# ---------------------------------------------------------------------------------------
def test_full_4096x4096_4bit_g64(O, dev):
    """The single-matrix workload, compared element by element over the whole tensor."""
    print("full 4096x4096", flush=True)
    W = weights(4096, 4096, 1_000_003, dev)
    out = run(W, 4, 64)
    compare(O, W, out, 4, 64, 16, label="4096x4096")


@pytest.mark.parametrize("rows,cols,nbits,g", [(11008, 4096, 4, 128), (4096, 11008, 2, 16),
                                               (13824, 5120, 2, 32), (8192, 28672, 3, 64)])
def test_full_size_sampled(O, dev, rows, cols, nbits, g):
    """Stack-sized tensors with 8-bit zeros: sampled groups against the oracle one by one
    (codes, scale and the binary32 zero are exact), the 8-bit zeros by their error bound."""
    print(f"full-size {rows}x{cols} b{nbits} g{g}", flush=True)
    W = weights(rows, cols, 31 * rows + cols + nbits, dev)
    out = run(W, nbits, g, zero_bits=8)
    ng = rows * cols // g
    idx = np.sort(RNG.choice(ng, 3000, replace=False))
    idx = np.unique(np.concatenate([idx, [0, ng - 1]]))
    w16 = u16(W).reshape(ng, g)
    sub = np.ascontiguousarray(w16[idx])
    ref = O.solve_groups(sub.reshape(-1), g, nbits)
    codes = O.unpack(u8(out["packed"]), rows * cols, nbits).reshape(ng, g)[idx]
    assert np.array_equal(codes.reshape(-1), ref["codes"])
    assert np.array_equal(u16(out["scale"])[idx], ref["scale"])
    z32 = out["workspace"][: 4 * ng].view(torch.float32).cpu().numpy()[idx]
    assert np.array_equal(z32, ref["zero_f32"])
    meta = u16(out["zero_meta"]).view(np.float16).astype(np.float64)
    zq = u8(out["zero"])[idx].astype(np.float64)
    zr = zq * meta[0] + meta[1]
    err = np.abs(zr - ref["zero_f32"])
    inner = (zq > 0) & (zq < 255)
    assert np.all(err[inner] <= 0.5 * meta[0] * (1 + 1e-5))      # half a step of the grid
    assert np.all(err <= (0.5 + 255 * 2.0 ** -11) * meta[0] + 2.0 ** -10 * abs(meta[1]))
    assert u8(out["zero"]).max() == 255 and u8(out["zero"]).min() == 0
    ok = ref["shrink_active"] == 0
    assert np.array_equal(u8(out["passes"])[idx][ok], ref["evals_needed"][ok])


def test_batch_equals_single_calls(O, dev):
    """One batched call over mixed jobs writes what the single-tensor calls write."""
    specs = [(256, 1024, 4, 64, 16), (512, 2048, 4, 128, 8), (128, 4096, 2, 16, 8),
             (64, 1280, 3, 64, 8), (96, 512, 2, 32, 16), (32, 256, 8, 16, 8)]
    Ws, outs, jobs = [], [], []
    for i, (r, c, b, g, zb) in enumerate(specs):
        W = weights(r, c, 900 + i, dev)
        o = hqq.alloc_outputs(r, c, b, g, zb, dev, passes=True)
        jobs.append(hqq.make_job(W, b, g, 1, 0.7, 1.0, 1.01, 20, 1, zb, o["packed"], o["scale"],
                                 o["zero"], o["zero_meta"], o["passes"]))
        Ws.append(W)
        outs.append(o)
    ws = hqq.alloc_workspace(jobs, dev)
    hqq.hqq_quantize_batch(jobs, ws)
    torch.cuda.synchronize()
    for W, o, (r, c, b, g, zb) in zip(Ws, outs, specs):
        single = run(W, b, g, zb)
        for k in ("packed", "scale", "zero", "passes"):
            assert torch.equal(o[k], single[k]), k
        if zb == 8:
            assert torch.equal(o["zero_meta"], single["zero_meta"])
        compare(O, W, o, b, g, zb, label=f"batch b{b} g{g}")


@pytest.mark.parametrize("layout", [1, 3, 0], ids=["persistent", "lockstep", "auto"])
def test_repeated_solves_are_identical(dev, layout):
    """The persistent solver claims tiles and moves groups between lanes in whatever order
    its waves reach them; the outputs must not depend on that order. The same mixed batch is
    solved five times over sentinel-filled outputs and every run must write the same bytes."""
    specs = [(4096, 4096, 4, 128, 8), (2048, 4096, 2, 16, 8), (1024, 2048, 3, 64, 8),
             (512, 4096, 4, 64, 16), (256, 1024, 8, 32, 16)]
    Ws, outs, jobs = [], [], []
    for i, (r, c, b, g, zb) in enumerate(specs):
        W = weights(r, c, 1700 + i, dev)
        o = hqq.alloc_outputs(r, c, b, g, zb, dev, passes=True)
        jobs.append(hqq.make_job(W, b, g, 1, 0.7, 1.0, 1.01, 20, 1, zb, o["packed"], o["scale"],
                                 o["zero"], o["zero_meta"], o["passes"]))
        Ws.append(W)
        outs.append(o)
    ws = hqq.alloc_workspace(jobs, dev)
    keys = ("packed", "scale", "zero", "passes")
    try:
        hqq.hqq_debug_solver(pass_layout=layout)
        first = None
        for run_i in range(5):
            print(f"repeat layout={layout} run {run_i}", flush=True)
            for o in outs:
                for k, v in zip(keys, (0x5A, 0, 0x33, 0xEE)):
                    o[k].view(torch.uint8).fill_(v)
            torch.cuda.synchronize()
            hqq.hqq_quantize_batch(jobs, ws)
            torch.cuda.synchronize()
            hqq.hqq_batch_check(jobs, ws)
            cur = [{k: o[k].clone() for k in keys + ("zero_meta",) if o[k] is not None} for o in outs]
            if first is None:
                first = cur
                continue
            for i, (a, b) in enumerate(zip(first, cur)):
                for k in a:
                    assert torch.equal(a[k], b[k]), f"run {run_i} tensor {i} {k} differs"
    finally:
        hqq.hqq_debug_solver()
