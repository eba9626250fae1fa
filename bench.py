#!/usr/bin/env python3
"""Throughput of the HQQ quantizer on one MI355X.

A step quantizes one whole Llama-2-7B-shaped stack (32 blocks x q,k,v,o,gate,up,down,
224 tensors, 6.48e9 binary16 weights resident in HBM; 4-bit, group 128, 8-bit zeros; see
--workload for the others) through the C ABI: the group solver over every tensor, then the
per-tensor 8-bit zero requantization. Prints one JSON line; beside the main line it measures
the other workloads, the stress input (beta0 = 1e4), the variants the pages describe and
the oracle on the host.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--oracle-all-core]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published peak
# Plain (non-packed) fp32 VALU issue rate: 64 lane operations per clock on each of the 256
# compute units at 2.4 GHz, 39.32e12/s. The published 157.3 TFLOP/s fp32 vector peak counts an
# FMA as two flops on packed two-lane instructions, which this library does not emit.
ALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12
METRIC = "fp16 weight GB/s quantized (% HBM peak); seconds per Llama-2-7B-shaped stack"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def alg_bytes(spec) -> float:
    """Algorithmic HBM bytes of one tensor: read binary16 weights once, write packed codes,
    binary16 scale and the zero (2 bytes, or 1 for 8-bit zeros) once per group."""
    from calibration_free_weight_amd import hqq
    n = spec.numel
    ng = n // spec.group_size
    zb = 2 if spec.zero_bits == 16 else 1
    return 2.0 * n + hqq.hqq_packed_bytes(n, spec.nbits) + ng * (2 + zb)


SOLVER_SOURCE = os.path.join(ROOT, "calibration_free_weight_amd", "csrc", "hqq_stream.hip")


def source_digest() -> str:
    import hashlib
    with open(SOLVER_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload: int):
    """HBM bytes per solver launch from the committed counter summary of this workload, or
    None when there is none or the solver source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_stream_kernel_workload{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("solver source sha256") != source_digest():
        return None
    return float(fields["hbm bytes per launch"])


def alg_ops_per_weight(mean_passes: float) -> float:
    """Algorithmic fp32 operations per weight: each evaluation of the quantizer costs 5 per
    element (fma, round, clamp; residual, absolute sum) and each zero update 3 (sub, fma,
    add); `mean_passes` counts evaluations, the first included."""
    return 5.0 * mean_passes + 3.0 * (mean_passes - 1.0)


def copy_probe(mib: int, dev):
    """A plain copy of known size (binary16 negation: reads and writes `mib` MiB once), run a
    few times so that a counter pass over this program can scale its byte counters."""
    import torch
    n = mib * (1 << 20) // 2
    a = torch.ones(n, dtype=torch.float16, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b


def cpu_baseline(block0, seconds):
    """The oracle, single-threaded, on a bounded sample of the same weights: leading rows of
    each distinct projection of block 0 (host copies), sized to about `seconds` of CPU work."""
    import oracle
    from synth import half_bits
    O = oracle.Oracle()
    # calibrate on a small slice, then size the sample
    s0, w0 = block0[0]
    probe_rows = max(1, 65536 // s0.cols)
    x = half_bits(w0[:probe_rows]).reshape(-1)
    t = time.perf_counter()
    O.solve_groups(x, s0.group_size, s0.nbits)
    rate = x.size / (time.perf_counter() - t)
    per_tensor = rate * seconds / len(block0)
    total_w, total_t, parts = 0, 0.0, []
    for s, w in block0:
        rows = int(max(1, min(w.shape[0], per_tensor // s.cols)))
        x = half_bits(w[:rows]).reshape(-1)
        t = time.perf_counter()
        O.quantize(x, s.group_size, s.nbits, zero_bits=s.zero_bits)
        total_t += time.perf_counter() - t
        total_w += x.size
        parts.append(f"{s.name}[:{rows}]")
    return dict(value=round(2.0 * total_w / total_t / 1e9, 6), unit="GB/s", cores=1,
                kind="oracle",
                sample=f"{total_w} weights ({', '.join(parts)}), one thread, "
                       f"{total_t:.1f} s; full quantize incl. zero storage and packing")


def scale8_row(dev, stream, reps=10):
    """8-bit scales in runs of 128 (the pages' HQQ_g16_s variant) on the scale array of a
    2-bit g16 Llama-2-7B-shaped stack: requant and read-back, each timed with HIP events on
    the launch stream over `reps` launches. Both are HBM-bound; algorithmic bytes per scale:
    requant 2 read + 1 written, read-back 1 read + 2 written, plus 4 per run of 128 (meta)."""
    import torch
    import synth
    from calibration_free_weight_amd import hqq
    n, group = 6_476_005_376 // 16, 128
    n_runs = (n + group - 1) // group
    v = synth.scale_values(n, 4711, device=dev)
    sq = torch.empty(n, dtype=torch.uint8, device=dev)
    meta = torch.empty(2 * n_runs, dtype=torch.float16, device=dev)
    back = torch.empty(n, dtype=torch.float16, device=dev)
    calls = {
        "requant": (lambda: hqq.hqq_requant_scales(v, n, group, sq, meta, stream.cuda_stream),
                    3 * n + 4 * n_runs, "scale_requant_kernel<16>"),
        "dequant": (lambda: hqq.hqq_dequantize_scales(sq, meta, n, group, back,
                                                      stream.cuda_stream),
                    3 * n + 4 * n_runs, "scale_dequant_kernel"),
    }
    row = {"variant": "8-bit scales, runs of 128 (HQQ_g16_s)", "n_scales": n, "bound": "hbm"}
    for name, (fn, nbytes, kern) in calls.items():
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbs = nbytes / (ms * 1e-3) / 1e9
        row[name] = {"kernel": kern, "launch_ms": round(ms, 4), "bytes_per_launch": nbytes,
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4)}
    del v, sq, meta, back
    return row


def axis0_row(specs, weights, dev, stream, axis1_solve_ms, reps=3):
    """The same stack with groups down columns (axis 0): the solve phase transposes each
    weight matrix (2 B read + 2 B written per weight) and runs the unchanged solver on the
    transposed copy; the requant phase writes codes and per-group arrays back in the
    tensor's order: packed codes transposed in one pass through LDS (nbits/4 B per weight;
    3-bit words take unpack, byte transpose and pack instead)."""
    import torch
    from calibration_free_weight_amd import hqq
    jobs, outs = [], []
    for s, w in zip(specs, weights):
        o = hqq.alloc_outputs(s.rows, s.cols, s.nbits, s.group_size, s.zero_bits, dev)
        jobs.append(hqq.make_job(w, s.nbits, s.group_size, 0, 0.7, 1.0, 1.01, 20, 1,
                                 s.zero_bits, o["packed"], o["scale"], o["zero"],
                                 o["zero_meta"]))
        outs.append(o)
    ws = hqq.alloc_workspace(jobs, dev)
    hqq.hqq_quantize_batch(jobs, ws, stream.cuda_stream)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for k in range(reps):
        ev[k][0].record(stream)
        hqq.hqq_solve_batch(jobs, ws, stream.cuda_stream)
        ev[k][1].record(stream)
        hqq.hqq_requant_batch(jobs, ws, stream.cuda_stream)
        ev[k][2].record(stream)
    torch.cuda.synchronize()
    solve = sum(e[0].elapsed_time(e[1]) for e in ev) / reps
    req = sum(e[1].elapsed_time(e[2]) for e in ev) / reps
    n = sum(s.numel for s in specs)
    glue = (solve - axis1_solve_ms) + req
    # W transpose 4 B; codes: one fused pass (nbits/4 B) where rows start on a byte, else
    # unpack + byte transpose + pack (4 + nbits/4 B); per-group arrays left out
    glue_bytes = sum(s.numel * (4 + s.nbits / 4 + (0 if s.nbits != 3 else 4)) for s in specs)
    del jobs, outs, ws
    return {"variant": "groups down columns (axis 0), same stack", "ms_per_stack": round(solve + req, 3),
            "value_gbs": round(2.0 * n / ((solve + req) * 1e-3) / 1e9, 1),
            "solve_phase_ms": round(solve, 3), "requant_phase_ms": round(req, 3),
            "axis1_solve_ms": round(axis1_solve_ms, 3), "glue_ms": round(glue, 3),
            "glue_bytes_per_weight": round(glue_bytes / n, 4), "bound": "hbm",
            "glue_achieved_gbs": round(glue_bytes / (glue * 1e-3) / 1e9, 1) if glue > 0 else None,
            "peak": HBM_PEAK_GBS}


def host_stream_row(specs, weights, dev, stream, reps=3):
    """The stack with its weights in pinned host memory (hqq_quantize_streamed: chunks of up
    to 1 GiB copied into a 2 GiB device staging buffer on a second stream while the previous
    chunk is solved). PCIe-inclusive: the copy of every weight is inside the timed region.
    Beside it, a plain host-to-device copy of the same bytes through the same staging."""
    import torch
    from calibration_free_weight_amd import hqq
    n = sum(s.numel for s in specs)
    pinned = torch.empty(n, dtype=torch.float16, pin_memory=True)
    jobs, outs, views, off = [], [], [], 0
    for s, w in zip(specs, weights):
        v = pinned[off:off + s.numel].view(s.rows, s.cols)
        v.copy_(w)
        o = hqq.alloc_outputs(s.rows, s.cols, s.nbits, s.group_size, s.zero_bits, dev)
        jobs.append(hqq.make_job(v, s.nbits, s.group_size, 1, 0.7, 1.0, 1.01, 20, 1,
                                 s.zero_bits, o["packed"], o["scale"], o["zero"],
                                 o["zero_meta"]))
        views.append(v)
        outs.append(o)
        off += s.numel
    staging_bytes = 2 << 30
    staging = torch.empty(staging_bytes, dtype=torch.uint8, device=dev)
    ws = torch.empty(max(hqq.hqq_streamed_workspace_bytes(jobs, staging_bytes), 256),
                     dtype=torch.uint8, device=dev)
    cs = torch.cuda.Stream()
    hqq.hqq_quantize_streamed(jobs, staging, ws, stream.cuda_stream, cs.cuda_stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        hqq.hqq_quantize_streamed(jobs, staging, ws, stream.cuda_stream, cs.cuda_stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    # the same bytes through the staging halves, copy only
    half = staging_bytes // 2
    st16 = staging.view(torch.float16)
    e0.record(stream)
    for _ in range(reps):
        used, h = 0, 0
        for v in views:
            if used + v.numel() * 2 > half:
                used, h = 0, 1 - h
            dst = st16[(h * half + used) // 2:(h * half + used) // 2 + v.numel()]
            dst.copy_(v.view(-1), non_blocking=True)
            used += (v.numel() * 2 + 255) // 256 * 256
    e1.record(stream)
    torch.cuda.synchronize()
    copy_ms = e0.elapsed_time(e1) / reps
    del jobs, outs, ws, staging, pinned, views
    return {"variant": "weights in pinned host memory, streamed (PCIe-inclusive)",
            "ms_per_stack": round(ms, 2), "value_gbs": round(2.0 * n / (ms * 1e-3) / 1e9, 1),
            "h2d_copy_only_ms": round(copy_ms, 2),
            "h2d_gbs": round(2.0 * n / (copy_ms * 1e-3) / 1e9, 1), "bound": "pcie",
            "peak": 64.0, "unit": "GB/s",
            "frac": round(2.0 * n / (ms * 1e-3) / 1e9 / 64.0, 4),
            "overlap": round(copy_ms / ms, 4)}


def dequant_row(specs, outs, dev, stream, reps=5):
    """hqq_dequantize (the layer's dequantize()) on the 224 quantized weights the benchmark
    just wrote: reads the packed codes, scales and 8-bit zeros, writes binary16 W_r; HBM-bound.
    One output buffer of the largest tensor's size serves every call."""
    import torch
    from calibration_free_weight_amd import hqq
    out = torch.empty(max(s.rows * s.cols for s in specs), dtype=torch.float16, device=dev)

    def run_all():
        for s, o in zip(specs, outs):
            hqq.hqq_dequantize(o["packed"], o["scale"], o["zero"], o["zero_meta"], s.rows,
                               s.cols, s.nbits, s.group_size, 1, s.zero_bits,
                               out[:s.rows * s.cols])
    run_all()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run_all()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = sum(o["packed"].numel() + o["scale"].numel() * 2 +
                 o["zero"].numel() * o["zero"].element_size() + 2 * s.rows * s.cols
                 for s, o in zip(specs, outs))
    gbs = nbytes / (ms * 1e-3) / 1e9
    del out
    return {"variant": "hqq_dequantize of every quantized weight of the stack (axis 1)",
            "ms_per_stack": round(ms, 4), "bytes": nbytes, "bound": "hbm",
            "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4)}


def fused_gemm_row(specs, outs, Xs, Ys, eager, stream, reps, nbytes, flops):
    """The same layers, with the projections that read one input multiplied by one
    hqq_gemm_multi call each (per block: q, k and v; gate and up; o and down alone), as an
    inference engine runs them: fewer, fuller launches. Graph-captured like the per-layer
    row and checked equal to its outputs."""
    import torch
    from calibration_free_weight_amd import hqq
    by_block = {}
    for s, o, Y in zip(specs, outs, Ys):
        by_block.setdefault(s.block, []).append((s, o, Y))
    calls = []
    for b in sorted(by_block):
        layers = sorted(by_block[b], key=lambda t: t[0].proj)
        for group in ((0, 1, 2), (3,), (4, 5), (6,)):
            members = [(s, o, Y) for s, o, Y in layers if s.proj in group]
            if members:
                weights = [dict(packed=o["packed"], scale=o["scale"], zero=o["zero"],
                                zero_meta=o["zero_meta"], N=s.rows, nbits=s.nbits,
                                group_size=s.group_size, zero_bits=s.zero_bits, Y=Y)
                           for s, o, Y in members]
                calls.append((Xs[members[0][0].cols], weights))

    def run_all():
        for X, weights in calls:
            hqq.hqq_gemm_multi(X, weights)
    for Y in Ys:
        Y.fill_(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all()
    for _ in range(2):
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(eager, Ys)), "fused layers differ"
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms_per_stack": round(ms, 4), "graph": True, "calls": len(calls),
            "hbm_gbs": round(gbs, 1), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4)}


def gemm_row(specs, outs, dev, stream, reps=5, graphs=True):
    """The quantized linear layers of the stack (hqq_gemm on the 224 quantized weights the
    benchmark just wrote). Decode, M = 1, and small batches, M = 16 and 64 (the weight
    streams once per call): the 224 calls are captured in a HIP graph (launch gaps would
    dominate otherwise) and the replay is checked against the eager result; rated against
    HBM on the bytes of packed weights, scales, zeros, X and Y. Prefill, M = 512: W_r
    reconstructed once per call into a workspace, then the binary16 matrix-core GEMM;
    2*M*N*K flops."""
    import torch
    from calibration_free_weight_amd import hqq
    kmax = max(s.cols for s in specs)
    res = {"variant": "quantized linear layers of the stack, Y = X . W_r^T"}
    for m in (1, 16, 64, 512):
        X = torch.randn(m, kmax, device=dev).to(torch.float16)
        Ys = [torch.empty(m, s.rows, dtype=torch.float16, device=dev) for s in specs]

        Xs = {c: X[:, :c].contiguous() for c in {s.cols for s in specs}}
        wb = max(hqq.hqq_gemm_workspace_bytes(m, s.rows, s.cols) for s in specs)
        ws = torch.empty(wb, dtype=torch.uint8, device=dev) if wb else None

        def run_all():
            for s, o, Y in zip(specs, outs, Ys):
                hqq.hqq_gemm(Xs[s.cols], o["packed"], o["scale"], o["zero"], o["zero_meta"],
                             s.rows, s.cols, s.nbits, s.group_size, s.zero_bits, Y,
                             workspace=ws)
        run_all()
        torch.cuda.synchronize()
        eager = [y.clone() for y in Ys]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        graphed = False
        if m <= 64 and graphs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_all()
            for _ in range(2):
                g.replay()
                torch.cuda.synchronize()
                assert all(torch.equal(a, b) for a, b in zip(eager, Ys)), "graph replay differs"
            graphed = True
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
        else:
            e0.record(stream)
            for _ in range(reps):
                run_all()
            e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        wbytes = sum(o["packed"].numel() + o["scale"].numel() * 2 +
                     o["zero"].numel() * o["zero"].element_size() for o in outs)
        nbytes = wbytes + sum(m * s.cols * 2 + m * s.rows * 2 for s in specs)
        flops = sum(2.0 * m * s.rows * s.cols for s in specs)
        row = {"m": m, "ms_per_stack": round(ms, 4), "graph": graphed,
               "workspace_bytes": wb,
               "bytes": nbytes, "flops": flops,
               "hbm_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
               "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
        if m <= 64:
            row.update(bound="hbm", achieved=row["hbm_gbs"], peak=HBM_PEAK_GBS, unit="GB/s",
                       frac=round(row["hbm_gbs"] / HBM_PEAK_GBS, 4))
        else:
            row.update(bound="mfma", achieved=row["tflops"], peak=2500.0, unit="TFLOP/s",
                       frac=round(row["tflops"] / 2500.0, 4))
        res[f"m{m}"] = row
        if m <= 64 and graphs:
            res[f"m{m}_fused"] = fused_gemm_row(specs, outs, Xs, Ys, eager, stream, reps, nbytes,
                                                flops)
        del X, Ys, eager, Xs, ws

    # Prefill with W_r resident: every layer's weight reconstructed once by hqq_dequantize
    # (13 GB for the 7B-shaped stack, well inside one GPU's HBM) and kept; each call is then
    # hqq_gemm_f16 alone. Checked equal to hqq_gemm's reconstruct-once path.
    m = 512
    X = torch.randn(m, kmax, device=dev).to(torch.float16)
    Xs = {c: X[:, :c].contiguous() for c in {s.cols for s in specs}}
    Ys = [torch.empty(m, s.rows, dtype=torch.float16, device=dev) for s in specs]
    wb = max(hqq.hqq_gemm_workspace_bytes(m, s.rows, s.cols) for s in specs)
    ws = torch.empty(wb, dtype=torch.uint8, device=dev)
    ref = [torch.empty_like(y) for y in Ys]
    wr = [torch.empty(s.rows, s.cols, dtype=torch.float16, device=dev) for s in specs]
    for s, o, Y, W in zip(specs, outs, ref, wr):
        hqq.hqq_gemm(Xs[s.cols], o["packed"], o["scale"], o["zero"], o["zero_meta"], s.rows,
                     s.cols, s.nbits, s.group_size, s.zero_bits, Y, workspace=ws,
                     stream=stream.cuda_stream)
        hqq.hqq_dequantize(o["packed"], o["scale"], o["zero"], o["zero_meta"], s.rows, s.cols,
                           s.nbits, s.group_size, 1, s.zero_bits, W, stream=stream.cuda_stream)

    def run_resident():
        for s, Y, W in zip(specs, Ys, wr):
            hqq.hqq_gemm_f16(Xs[s.cols], W, s.rows, s.cols, Y, stream=stream.cuda_stream)

    run_resident()
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(Ys, ref)), "hqq_gemm_f16 differs from hqq_gemm"
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run_resident()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = sum(2.0 * m * s.rows * s.cols for s in specs)
    tf = round(flops / (ms * 1e-3) / 1e12, 2)
    res["m512_resident"] = {"m": m, "ms_per_stack": round(ms, 4), "graph": False,
                            "variant": "hqq_gemm_f16 on W_r reconstructed once by "
                                       "hqq_dequantize and kept resident",
                            "resident_bytes": sum(2 * s.rows * s.cols for s in specs),
                            "flops": flops, "tflops": tf, "bound": "mfma", "achieved": tf,
                            "peak": 2500.0, "unit": "TFLOP/s", "frac": round(tf / 2500.0, 4)}
    del X, Xs, Ys, ws, ref, wr
    return res


def build_workload(number, dev, beta=1.0, sets=1):
    """Weights of a workload resident in HBM, preallocated outputs and a workspace. With
    sets > 1 (the single-matrix workload, which fits the 256 MB last-level cache) that many
    input/output sets are made so that consecutive launches stream from HBM."""
    import synth
    from calibration_free_weight_amd import hqq
    specs = synth.workload(number)
    weights, outs, job_sets, keep = [], [], [], []
    for r in range(sets):
        js = []
        for s in specs:
            seed = s.seed(number) + 7919 * r
            w = synth.student_t_weights(s.rows, s.cols, seed, device=dev)
            o = hqq.alloc_outputs(s.rows, s.cols, s.nbits, s.group_size, s.zero_bits, dev)
            js.append(hqq.make_job(w, s.nbits, s.group_size, 1, 0.7, beta, 1.01, 20, 1,
                                   s.zero_bits, o["packed"], o["scale"], o["zero"],
                                   o["zero_meta"]))
            if r == 0:
                weights.append(w)
                outs.append(o)
            else:
                keep.append((w, o))
        job_sets.append(js)
    ws = hqq.alloc_workspace(job_sets[0], dev)
    return dict(specs=specs, weights=weights, outs=outs, job_sets=job_sets, ws=ws, keep=keep)


def time_steps(wl, stream, steps, warmup):
    """Runs `steps` steps (solve, then requant) after `warmup` untimed ones, rotating over the
    workload's sets. Returns the wall seconds of the timed steps and the per-step solver and
    requant times in ms from HIP events on the launch stream."""
    import torch
    from calibration_free_weight_amd import hqq
    js_all, ws = wl["job_sets"], wl["ws"]
    for i in range(warmup):
        hqq.hqq_quantize_batch(js_all[i % len(js_all)], ws, stream.cuda_stream)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        js = js_all[k % len(js_all)]
        ev[k][0].record(stream)
        hqq.hqq_solve_batch(js, ws, stream.cuda_stream)
        ev[k][1].record(stream)
        hqq.hqq_requant_batch(js, ws, stream.cuda_stream)
        ev[k][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    hqq.hqq_batch_check(js_all[(steps - 1) % len(js_all)], ws, stream.cuda_stream)
    solve = [e[0].elapsed_time(e[1]) for e in ev]
    req = [e[1].elapsed_time(e[2]) for e in ev]
    return wall, solve, req


def mean_passes(wl, stream, dev):
    """Mean evaluations per group, from the solver's own per-group counts: one more (untimed)
    solve of the first set with the count outputs set."""
    import torch
    from calibration_free_weight_amd import hqq
    counts = []
    for s, j in zip(wl["specs"], wl["job_sets"][0]):
        pb = torch.empty(s.numel // s.group_size, dtype=torch.uint8, device=dev)
        j.passes = pb.data_ptr()
        counts.append(pb)
    hqq.hqq_solve_batch(wl["job_sets"][0], wl["ws"], stream.cuda_stream)
    torch.cuda.synchronize()
    n_pass = sum(int(pb.sum(dtype=torch.int64).item()) for pb in counts)
    n_groups = sum(pb.numel() for pb in counts)
    for j in wl["job_sets"][0]:
        j.passes = None
    return n_pass / n_groups


def roofline(specs, solve_ms, passes):
    """Both roofs of the solver launches: algorithmic HBM bytes and algorithmic fp32 lane
    operations per launch (one launch per class of tensors sharing bit width and group size)
    over the median launch time; the binding roof is the one with the longer floor."""
    classes = sorted({(s.nbits, s.group_size) for s in specs})
    launches = len(classes)
    n_weights = sum(s.numel for s in specs)
    launch_s = solve_ms * 1e-3 / launches
    bytes_launch = sum(alg_bytes(s) for s in specs) / launches
    ops_launch = n_weights * alg_ops_per_weight(passes) / launches
    hbm = {"achieved": round(bytes_launch / launch_s / 1e9, 2), "peak": HBM_PEAK_GBS,
           "unit": "GB/s", "floor_ms": round(bytes_launch / HBM_PEAK_GBS / 1e6, 4)}
    hbm["frac"] = round(hbm["achieved"] / HBM_PEAK_GBS, 4)
    alu = {"achieved": round(ops_launch / launch_s / 1e12, 3), "peak": round(ALU_PEAK_TOPS, 3),
           "unit": "Top/s", "floor_ms": round(ops_launch / ALU_PEAK_TOPS / 1e9, 4)}
    alu["frac"] = round(alu["achieved"] / ALU_PEAK_TOPS, 4)
    bound, main = ("alu", alu) if alu["floor_ms"] > hbm["floor_ms"] else ("hbm", hbm)
    # The library runs a class on the lockstep kernel when it has fewer than about four groups
    # per lane of the persistent grid (256 compute units x 12 waves x 64 lanes), else on the
    # persistent one.
    def kernel_name(b, g):
        groups = sum(s.numel // s.group_size for s in specs if (s.nbits, s.group_size) == (b, g))
        small = groups < 4 * 256 * 12 * 64
        return f"{'lockstep_kernel' if small else 'stream_kernel'}<{b},{g}>"
    return {"bound": bound,
            "kernel": ", ".join(kernel_name(b, g) for b, g in classes),
            "achieved": main["achieved"], "peak": main["peak"], "unit": main["unit"],
            "frac": main["frac"], "launch_ms": round(launch_s * 1e3, 5),
            "bytes_per_launch": round(bytes_launch, 1), "ops_per_launch": round(ops_launch, 1),
            "mean_passes": round(passes, 4), "hbm": hbm, "alu": alu}


def config_row(number, dev, stream, steps, beta=1.0, sets=1):
    """One workload measured like the main line: seconds per stack (median over the steps of
    solve + requant, HIP events), binary16 GB/s quantized, and the solver's roofs."""
    import statistics
    import synth
    wl = build_workload(number, dev, beta=beta, sets=sets)
    _, solve, req = time_steps(wl, stream, steps, warmup=2)
    passes = mean_passes(wl, stream, dev)
    n = sum(s.numel for s in wl["specs"])
    step_ms = statistics.median(a + b for a, b in zip(solve, req))
    row = {"workload": synth.WORKLOAD_NAMES[number], "beta": beta, "weights": n,
           "steps": steps, "sets": sets, "ms_per_stack": round(step_ms, 4),
           "value_gbs": round(2.0 * n / (step_ms * 1e-3) / 1e9, 1),
           "solve_ms_median": round(statistics.median(solve), 4),
           "requant_ms_median": round(statistics.median(req), 4),
           "pct_hbm_peak": round(100.0 * sum(alg_bytes(s) for s in wl["specs"]) /
                                 (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 3),
           "roofline": roofline(wl["specs"], statistics.median(solve), passes)}
    del wl
    return row


def oracle_all_core(wl, stream):
    """The whole stack through the oracle on P single-threaded processes (one per host core,
    at most 16), tensor by tensor, each result compared with what the GPU wrote. Reports the
    wall time of the oracle with P stated."""
    import numpy as np
    import torch
    import oracle
    from oracle.pool import OraclePool
    from calibration_free_weight_amd import hqq
    O = oracle.Oracle()
    hqq.hqq_quantize_batch(wl["job_sets"][0], wl["ws"], stream.cuda_stream)
    torch.cuda.synchronize()
    n_w, t_oracle, mismatches = 0, 0.0, 0
    with OraclePool() as pool:
        for s, w, o in zip(wl["specs"], wl["weights"], wl["outs"]):
            w16 = w.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
            t = time.perf_counter()
            ref = pool.solve_groups(w16.reshape(-1), s.group_size, s.nbits)
            t_oracle += time.perf_counter() - t
            n_w += s.numel
            packed = o["packed"].cpu().numpy()
            mismatches += int(not np.array_equal(packed[:O.packed_bytes(s.numel, s.nbits)],
                                                 O.pack(ref["codes"], s.nbits)))
            zq, meta = O.zero_requant(ref["zero_f32"])
            mismatches += int(not np.array_equal(o["zero"].cpu().numpy(), zq))
            mismatches += int(not np.array_equal(
                o["scale"].cpu().view(torch.int16).numpy().view(np.uint16), ref["scale"]))
            if s.proj == 6:
                log(f"bench: oracle on block {s.block} done ({t_oracle:.0f} s)")
        procs = pool.procs
    return {"kind": "oracle", "procs": procs, "weights": n_w, "wall_s": round(t_oracle, 2),
            "value": round(2.0 * n_w / t_oracle / 1e9, 5), "unit": "GB/s",
            "tensors_differing": mismatches,
            "note": "oracle (single-threaded C) in P processes over the tensor's groups; "
                    "wall time of the solves only, host copies excluded"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-next-rows", action="store_true",
                    help="only the main step (for a kernel trace of the solver alone)")
    ap.add_argument("--rows", default="scale8,axis0,dequant,gemm,host_stream,configs",
                    help="which rows beside the main line to measure (comma-separated)")
    ap.add_argument("--gemm-eager", action="store_true",
                    help="launch the small-batch GEMM rows eagerly, not from HIP graphs (for "
                         "counter passes)")
    ap.add_argument("--oracle-all-core", action="store_true",
                    help="also run the oracle over the whole workload on every host core "
                         "(minutes) and compare it with the GPU")
    ap.add_argument("--beta", type=float, default=1.0,
                    help="beta0 of the main line (1e4 makes the shrink live: stress input)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run a plain copy of this many MiB first (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the quantizer shards by whole tensors with no communication)", file=sys.stderr)
        sys.exit(2)

    import statistics
    import torch
    import synth

    dev = torch.device("cuda:0")
    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib, dev)
    stream = torch.cuda.current_stream()
    log(f"bench: workload {args.workload} ({synth.WORKLOAD_NAMES[args.workload]})")
    # Inputs resident in HBM; outputs and workspace preallocated. The single-matrix workload
    # rotates 16 sets (512 MiB of inputs) so that every step streams from HBM.
    wl = build_workload(args.workload, dev, beta=args.beta,
                        sets=16 if args.workload == 1 else 1)
    specs, weights, outs = wl["specs"], wl["weights"], wl["outs"]
    n_weights = sum(s.numel for s in specs)
    log(f"bench: {len(specs)} tensors, {n_weights / 1e9:.3f}e9 weights ready")
    cpu_input = None
    if not args.no_cpu_baseline:             # host copy of the oracle's sample, taken now
        cpu_input = [(s, w[:max(1, min(s.rows, 12_000_000 // s.cols))].cpu())
                     for s, w in zip(specs, weights) if s.block == 0]

    steps = max(args.steps, 200) if args.workload == 1 else args.steps
    wall, solve, req = time_steps(wl, stream, steps, args.warmup)
    log("bench: timed steps done")
    passes = mean_passes(wl, stream, dev)
    sec_per_step = wall / steps
    value = 2.0 * n_weights / sec_per_step / 1e9
    solve_ms = statistics.median(solve)
    bytes_step = sum(alg_bytes(s) for s in specs)
    roof = roofline(specs, solve_ms, passes)
    roof["launch_ms_mean"] = round(statistics.mean(solve) / len(roof["kernel"].split(", ")), 5)
    roof["traffic"] = measured_traffic(args.workload)
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec_per_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32+f64",
        "data": "synthetic",
        "config": {"workload": synth.WORKLOAD_NAMES[args.workload], "tensors": len(specs),
                   "weights": n_weights, "p": 0.7, "beta": args.beta, "kappa": 1.01,
                   "iters": 20, "early_stop": True},
        "seconds_per_stack": round(sec_per_step, 6),
        "seconds_per_stack_median_events": round(
            statistics.median(a + b for a, b in zip(solve, req)) * 1e-3, 6),
        "pct_hbm_peak": round(100.0 * bytes_step / sec_per_step / 1e9 / HBM_PEAK_GBS, 3),
        "roofline": roof,
    }
    want = set() if args.skip_next_rows else set(args.rows.split(","))
    result["next_rows"] = {}
    if "scale8" in want:
        log("bench: 8-bit scales")
        result["next_rows"]["scale8"] = scale8_row(dev, stream)
    if args.workload == 2 and "axis0" in want:
        log("bench: axis 0")
        result["next_rows"]["axis0"] = axis0_row(specs, weights, dev, stream, solve_ms)
    if args.workload == 2 and "dequant" in want:
        log("bench: dequantize")
        result["next_rows"]["dequant"] = dequant_row(specs, outs, dev, stream)
    if args.workload == 2 and "gemm" in want:
        log("bench: quantized linear layers")
        result["next_rows"]["gemm"] = gemm_row(specs, outs, dev, stream,
                                               graphs=not args.gemm_eager)
    if args.workload == 2 and "host_stream" in want:
        log("bench: host streaming")
        result["next_rows"]["host_stream"] = host_stream_row(specs, weights, dev, stream)
    if args.oracle_all_core:
        log("bench: the oracle over the whole workload on every host core")
        result["oracle_all_core"] = oracle_all_core(wl, stream)
        result["oracle_all_core"]["gpu_speedup"] = round(
            result["oracle_all_core"]["wall_s"] / sec_per_step, 1)
    del wl, specs, weights, outs
    torch.cuda.empty_cache()
    if args.workload == 2 and "configs" in want:
        # the other workloads, each measured like the main line (config 1 over 16 rotating
        # sets, 256 launches), and the stress input (config 1 with beta0 = 1e4: the shrink
        # and its pow are live in most groups)
        rows = {}
        for number, steps_w, sets in ((1, 256, 16), (3, 5, 1), (4, 5, 1), (5, 3, 1)):
            log(f"bench: workload {number}")
            rows[f"workload{number}"] = config_row(number, dev, stream, steps_w, sets=sets)
            torch.cuda.empty_cache()
        log("bench: stress input")
        rows["stress_beta1e4"] = config_row(1, dev, stream, 256, beta=1e4, sets=16)
        result["next_rows"]["configs"] = rows
    if cpu_input is not None:
        log("bench: timing the oracle on the host")
        result["cpu_baseline"] = cpu_baseline(cpu_input, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
