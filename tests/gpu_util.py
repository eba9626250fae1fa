"""Helpers for the GPU parity tests: run the HIP path through the C ABI and compare it with
the oracle on the same binary16 bytes."""
from __future__ import annotations

import numpy as np
import torch

import synth


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16).reshape(-1)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().reshape(-1)


def weights(rows, cols, seed, dev):
    """Seeded synthetic weights generated on the device (fast at any size)."""
    return synth.student_t_weights(rows, cols, seed, device=dev)


# Spec tolerances of the HIP path against the oracle.
CODE_FRAC = 1e-4       # at most this fraction of codes may differ, each by at most 1
REL = 1e-3             # scale and zero, relative (zero: relative to max(|z|, 1 code step))
MSE_REL = 1e-3         # per-tensor reconstruction MSE


def compare(O, W, out, nbits, g, zero_bits, exact=True, params=None, label=""):
    """Compare the HIP outputs with the oracle for a whole tensor.

    exact=True asserts bit equality of codes, packed bytes, scale, zero (and meta) and of the
    evaluation counts; it always asserts the documented tolerances too. Returns the oracle
    result."""
    params = params or {}
    w16 = u16(W)
    ref = O.quantize(w16, g, nbits, zero_bits=zero_bits, **params)
    n = w16.size
    packed = u8(out["packed"])[:ref["packed"].size]
    codes = O.unpack(packed, n, nbits)
    scale = u16(out["scale"])
    zero = u16(out["zero"]) if zero_bits == 16 else u8(out["zero"])
    # --- tolerance bar ---
    dc = np.abs(codes.astype(np.int32) - ref["codes"].astype(np.int32))
    assert dc.max(initial=0) <= 1, f"{label}: a code differs by more than 1"
    assert (dc > 0).mean() <= CODE_FRAC, f"{label}: {(dc > 0).mean():.2e} of codes differ"
    s_g = scale.view(np.float16).astype(np.float64)
    s_r = ref["scale"].view(np.float16).astype(np.float64)
    assert np.all(np.abs(s_g - s_r) <= REL * np.abs(s_r)), f"{label}: scale"
    meta = None
    if zero_bits == 16:
        z_g = zero.view(np.float16).astype(np.float64)
        z_r = ref["zero"].view(np.float16).astype(np.float64)
        bad = np.abs(z_g - z_r) > REL * np.maximum(np.abs(z_r), 1.0)
        assert not bad.any(), f"{label}: {bad.sum()} zeros outside tolerance"
    else:
        meta = u16(out["zero_meta"])
        dz = np.abs(zero.astype(np.int32) - ref["zero"].astype(np.int32))
        assert dz.max(initial=0) <= 1, f"{label}: 8-bit zero differs by more than 1"
        m_g = meta.view(np.float16).astype(np.float64)
        m_r = ref["zero_meta"].view(np.float16).astype(np.float64)
        assert np.all(np.abs(m_g - m_r) <= REL * np.maximum(np.abs(m_r), 1e-3)), f"{label}: meta"
    mse_g = O.mse(w16, codes, scale, zero, meta, g, zero_bits)
    mse_r = O.mse(w16, ref["codes"], ref["scale"], ref["zero"], ref["zero_meta"], g, zero_bits)
    assert abs(mse_g - mse_r) <= MSE_REL * mse_r + 1e-30, f"{label}: mse {mse_g} vs {mse_r}"
    # --- exactness claim (binary64-exact per-element arithmetic on both sides) ---
    if exact:
        nd = int((codes != ref["codes"]).sum())
        assert nd == 0, f"{label}: {nd} codes differ"
        assert np.array_equal(packed, ref["packed"]), f"{label}: packed bytes differ"
        assert np.array_equal(scale, ref["scale"]), f"{label}: scale bits differ"
        assert np.array_equal(zero, ref["zero"]), \
            f"{label}: {(zero != ref['zero']).sum()} zeros differ"
        if zero_bits == 8:
            assert np.array_equal(meta, ref["zero_meta"]), f"{label}: meta bits differ"
        if out.get("passes") is not None:
            ok = ref["shrink_active"] == 0
            got = u8(out["passes"])
            assert np.array_equal(got[ok], ref["evals_needed"][ok]), \
                f"{label}: {(got[ok] != ref['evals_needed'][ok]).sum()} pass counts differ"
    return ref


def compare_whole(O, pool, W, out, nbits, g, zero_bits, zero32=None, label=""):
    """Element-by-element comparison of one whole tensor's outputs with the oracle, its
    groups solved by `pool` (the single-threaded oracle in several processes): packed
    bytes, scales, zeros (binary16, or uint8 codes and their binary16 step/base), the
    binary32 zeros when `zero32` is given, and the evaluation counts of groups whose shrink
    stayed dead. Returns the oracle result."""
    w16 = u16(W)
    n = w16.size
    ng = n // g
    ref = pool.solve_groups(w16, g, nbits)
    nb = O.packed_bytes(n, nbits)
    packed = u8(out["packed"])[:nb]
    ref_packed = O.pack(ref["codes"], nbits)
    if not np.array_equal(packed, ref_packed):
        codes = O.unpack(packed, n, nbits)
        bad = np.flatnonzero(codes != ref["codes"])
        raise AssertionError(f"{label}: {bad.size} of {n} codes differ (first at {bad[:5]})")
    scale = u16(out["scale"])
    assert np.array_equal(scale, ref["scale"]), \
        f"{label}: {(scale != ref['scale']).sum()} scales differ"
    if zero32 is not None:
        z32 = zero32.detach().cpu().numpy().reshape(-1)[:ng]
        assert np.array_equal(z32.view(np.uint32), ref["zero_f32"].view(np.uint32)), \
            f"{label}: {(z32 != ref['zero_f32']).sum()} binary32 zeros differ"
    if zero_bits == 16:
        zero = u16(out["zero"])
        assert np.array_equal(zero, O.zero_to_half(ref["zero_f32"])), f"{label}: zeros differ"
    else:
        zq, meta = O.zero_requant(ref["zero_f32"])
        got = u8(out["zero"])
        assert np.array_equal(got, zq), f"{label}: {(got != zq).sum()} 8-bit zeros differ"
        assert np.array_equal(u16(out["zero_meta"]), meta), f"{label}: zero meta differs"
    if out.get("passes") is not None:
        ok = ref["shrink_active"] == 0
        got = u8(out["passes"])
        assert np.array_equal(got[ok], ref["evals_needed"][ok]), \
            f"{label}: {(got[ok] != ref['evals_needed'][ok]).sum()} evaluation counts differ"
    return ref
