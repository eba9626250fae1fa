"""ctypes front end of the C oracle (test infrastructure, see the package docstring)."""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hqq_oracle.c")
_LIB = os.path.join(_HERE, "libhqq_oracle.so")

# One rounding per written operation: no contraction of a*b+c into fma, no fast-math, no
# vectoriser reassociation (gcc only reassociates under -ffast-math), no OpenMP.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra"]


def lib_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/libhqq_oracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_vp = C.c_void_p


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


class Oracle:
    """Handle on the compiled oracle. Arrays in and out are numpy."""

    def __init__(self, path: str | None = None):
        path = path or _LIB
        if not os.path.exists(path):
            build(force=False)
        L = C.CDLL(path)
        L.hqo_half_to_float.restype = C.c_float
        L.hqo_half_to_float.argtypes = [C.c_uint16]
        L.hqo_float_to_half.restype = C.c_uint16
        L.hqo_float_to_half.argtypes = [C.c_float]
        L.hqo_shrink.restype = C.c_double
        L.hqo_shrink.argtypes = [C.c_double, C.c_float, C.c_float]
        L.hqo_zero_update.restype = C.c_float
        L.hqo_zero_update.argtypes = [_f64p, _f64p, _f64p, C.c_float, C.c_int]
        L.hqo_eval.restype = C.c_double
        L.hqo_eval.argtypes = [_f64p, C.c_int, C.c_float, C.c_float, C.c_int, _f64p, _f64p]
        L.hqo_init.restype = None
        L.hqo_init.argtypes = [_f64p, C.c_int, C.c_int, C.POINTER(C.c_float),
                               C.POINTER(C.c_float)]
        L.hqo_solve_group.restype = C.c_double
        L.hqo_solve_group.argtypes = [_f64p, C.c_int, C.c_int, C.c_float, C.c_float, C.c_float,
                                      C.c_int, C.c_int, _u8p, C.POINTER(C.c_float),
                                      C.POINTER(C.c_float), C.POINTER(C.c_int),
                                      C.POINTER(C.c_int), C.POINTER(C.c_int),
                                      C.POINTER(C.c_int), _vp, _vp]
        L.hqo_solve_groups.restype = None
        L.hqo_solve_groups.argtypes = [_u16p, C.c_int64, C.c_int, C.c_int, C.c_float, C.c_float,
                                       C.c_float, C.c_int, C.c_int, _u8p, _u16p, _f32p, _vp,
                                       _vp, _vp, _vp, _vp]
        L.hqo_zero_requant.restype = None
        L.hqo_zero_requant.argtypes = [_f32p, C.c_int64, _u8p, _u16p]
        L.hqo_u8_affine.restype = None
        L.hqo_u8_affine.argtypes = [_f32p, C.c_int64, _u8p, _u16p]
        L.hqo_scale_requant.restype = None
        L.hqo_scale_requant.argtypes = [_u16p, C.c_int64, C.c_int, _u8p, _u16p]
        L.hqo_scale_dequant.restype = None
        L.hqo_scale_dequant.argtypes = [_u8p, _u16p, C.c_int64, C.c_int, _u16p]
        L.hqo_zero_to_half.restype = None
        L.hqo_zero_to_half.argtypes = [_f32p, C.c_int64, _u16p]
        L.hqo_packed_bytes.restype = C.c_size_t
        L.hqo_packed_bytes.argtypes = [C.c_int64, C.c_int]
        L.hqo_pack.restype = None
        L.hqo_pack.argtypes = [_u8p, C.c_int64, C.c_int, _u8p]
        L.hqo_unpack.restype = None
        L.hqo_unpack.argtypes = [_u8p, C.c_int64, C.c_int, _u8p]
        L.hqo_dequantize.restype = None
        L.hqo_dequantize.argtypes = [_u8p, _u16p, _vp, _vp, C.c_int64, C.c_int, C.c_int, _u16p]
        L.hqo_mse.restype = C.c_double
        L.hqo_mse.argtypes = [_u16p, _u8p, _u16p, _vp, _vp, C.c_int64, C.c_int, C.c_int]
        self.L = L

    # ---- scalar helpers --------------------------------------------------------------
    def half_to_float(self, h: int) -> float:
        return float(self.L.hqo_half_to_float(int(h)))

    def float_to_half(self, f: float) -> int:
        return int(self.L.hqo_float_to_half(float(np.float32(f))))

    def shrink(self, r: float, p: float, beta: float) -> float:
        return float(self.L.hqo_shrink(r, p, beta))

    def zero_update(self, x, q, we, s) -> float:
        x = np.ascontiguousarray(x, np.float64)
        q = np.ascontiguousarray(q, np.float64)
        we = np.ascontiguousarray(we, np.float64)
        return float(self.L.hqo_zero_update(x, q, we, s, len(x)))

    def eval(self, x, s, z, nbits):
        """Returns (S, q, r): S = sum |x*s + z - q| (exact), codes, residuals x - W_r."""
        x = np.ascontiguousarray(x, np.float64)
        q = np.empty_like(x)
        r = np.empty_like(x)
        S = self.L.hqo_eval(x, len(x), s, z, (1 << nbits) - 1, q, r)
        return float(S), q, r

    def init(self, x, nbits):
        x = np.ascontiguousarray(x, np.float64)
        s = C.c_float()
        z = C.c_float()
        self.L.hqo_init(x, len(x), (1 << nbits) - 1, C.byref(s), C.byref(z))
        return float(s.value), float(z.value)

    # ---- one group with its trace -------------------------------------------------------
    def solve_group(self, x, nbits, p=0.7, beta=1.0, kappa=1.01, iters=20, early_stop=1):
        """x: the group's values (binary16-representable), as float64."""
        x = np.ascontiguousarray(x, np.float64)
        g = len(x)
        codes = np.empty(g, np.uint8)
        s = C.c_float()
        z = C.c_float()
        np_ = C.c_int()
        lc = C.c_int()
        act = C.c_int()
        rose = C.c_int()
        te = np.zeros(iters + 1, np.float64)
        ta = np.zeros(iters + 1, np.uint8)
        e = self.L.hqo_solve_group(x, g, nbits, p, beta, kappa, iters, early_stop, codes,
                                   C.byref(s), C.byref(z), C.byref(np_), C.byref(lc),
                                   C.byref(act), C.byref(rose), _ptr(te), _ptr(ta))
        n = np_.value
        return dict(codes=codes, s=float(s.value), z=float(z.value), passes=n,
                    last_change=lc.value, shrink_active=act.value, stopped=rose.value,
                    err=float(e),
                    trace_S=te[:n].copy(), trace_acc=ta[:n].copy())

    # ---- many groups / tensors -------------------------------------------------------------
    def solve_groups(self, w16, g, nbits, p=0.7, beta=1.0, kappa=1.01, iters=20, early_stop=1):
        """w16: uint16 binary16 bit patterns, length a multiple of g (groups are consecutive)."""
        w16 = np.ascontiguousarray(w16, np.uint16).reshape(-1)
        assert w16.size % g == 0
        ng = w16.size // g
        out = dict(codes=np.empty(w16.size, np.uint8), scale=np.empty(ng, np.uint16),
                   zero_f32=np.empty(ng, np.float32), s=np.empty(ng, np.float32),
                   passes=np.empty(ng, np.uint8), last_change=np.empty(ng, np.uint8),
                   shrink_active=np.empty(ng, np.uint8), stopped=np.empty(ng, np.uint8))
        self.L.hqo_solve_groups(w16, ng, g, nbits, p, beta, kappa, iters, early_stop,
                                out["codes"], out["scale"], out["zero_f32"], _ptr(out["s"]),
                                _ptr(out["passes"]), _ptr(out["last_change"]),
                                _ptr(out["shrink_active"]), _ptr(out["stopped"]))
        # Evaluations needed by a solver that leaves a group once its zero repeats exactly
        # (every later iteration would be identical): all of them if the loop ended on a
        # rise, else one per change of the zero plus the initial one.
        out["evals_needed"] = np.where(out["stopped"] == 1, out["passes"],
                                       out["last_change"].astype(np.int32) + 1).astype(np.uint8)
        return out

    def zero_requant(self, z):
        z = np.ascontiguousarray(z, np.float32).reshape(-1)
        zq = np.empty(z.size, np.uint8)
        meta = np.empty(2, np.uint16)
        self.L.hqo_zero_requant(z, z.size, zq, meta)
        return zq, meta

    def u8_affine(self, v):
        """One min-max affine uint8 quantizer over all of v: (codes, meta {step, base})."""
        v = np.ascontiguousarray(v, np.float32).reshape(-1)
        q = np.empty(v.size, np.uint8)
        meta = np.empty(2, np.uint16)
        self.L.hqo_u8_affine(v, v.size, q, meta)
        return q, meta

    def scale_requant(self, scale16, group=128):
        """8-bit scales: binary16 scales (uint16 bits) -> (codes, meta [2*groups])."""
        scale16 = np.ascontiguousarray(scale16, np.uint16).reshape(-1)
        n = scale16.size
        sq = np.empty(n, np.uint8)
        meta = np.empty(2 * ((n + group - 1) // group), np.uint16)
        if n:
            self.L.hqo_scale_requant(scale16, n, group, sq, meta)
        return sq, meta

    def scale_dequant(self, sq, meta, group=128):
        """binary16 scales (uint16 bits) read back from 8-bit scales."""
        sq = np.ascontiguousarray(sq, np.uint8).reshape(-1)
        meta = np.ascontiguousarray(meta, np.uint16).reshape(-1)
        out = np.empty(sq.size, np.uint16)
        if sq.size:
            self.L.hqo_scale_dequant(sq, meta, sq.size, group, out)
        return out

    def zero_to_half(self, z):
        z = np.ascontiguousarray(z, np.float32).reshape(-1)
        zh = np.empty(z.size, np.uint16)
        self.L.hqo_zero_to_half(z, z.size, zh)
        return zh

    def quantize(self, w16, group_size, nbits, p=0.7, beta=1.0, kappa=1.01, iters=20,
                 early_stop=1, zero_bits=16):
        """Whole tensor (row-major, groups along axis 1): solver + zero storage + packing."""
        w16 = np.ascontiguousarray(w16, np.uint16)
        r = self.solve_groups(w16, group_size, nbits, p, beta, kappa, iters, early_stop)
        if zero_bits == 16:
            r["zero"] = self.zero_to_half(r["zero_f32"])
            r["zero_meta"] = None
        else:
            r["zero"], r["zero_meta"] = self.zero_requant(r["zero_f32"])
        r["packed"] = self.pack(r["codes"], nbits)
        return r

    def quantize_axis0(self, w16, rows, cols, group_size, nbits, p=0.7, beta=1.0, kappa=1.01,
                       iters=20, early_stop=1, zero_bits=16):
        """Whole tensor with groups down the columns (axis 0) [SK "Quantization configuration",
        axis]. Reading: group (b, j) is W[b*g:(b+1)*g, j]; the per-group solver is unchanged.
        Per-group outputs (scale, zero, s, passes, ...) form a [rows/g, cols] row-major array,
        group (b, j) at b*cols + j; the codes stay in the tensor's row-major order, so the
        packed stream has the same layout as for axis 1. The 8-bit zero grid is per tensor
        (order-independent)."""
        assert rows % group_size == 0
        w = np.ascontiguousarray(w16, np.uint16).reshape(rows, cols)
        cg = np.ascontiguousarray(w.T)                     # column j's runs, one after another
        r = self.solve_groups(cg.reshape(-1), group_size, nbits, p, beta, kappa, iters,
                              early_stop)
        nb = rows // group_size
        out = {}
        for k, v in r.items():                             # per group: [cols, nb] -> [nb, cols]
            out[k] = np.ascontiguousarray(v.reshape(cols, nb).T).reshape(-1) if k != "codes" \
                else np.ascontiguousarray(v.reshape(cols, rows).T).reshape(-1)
        if zero_bits == 16:
            out["zero"] = self.zero_to_half(out["zero_f32"])
            out["zero_meta"] = None
        else:
            out["zero"], out["zero_meta"] = self.zero_requant(out["zero_f32"])
        out["packed"] = self.pack(out["codes"], nbits)
        return out

    def dequantize_axis0(self, codes, scale, zero, zero_meta, rows, cols, g, zero_bits):
        """Reconstruction for axis 0: W_r[i, j] from group (i//g, j)'s scale and zero."""
        rep = lambda a: np.ascontiguousarray(
            np.repeat(np.asarray(a).reshape(rows // g, cols), g, axis=0)).reshape(-1)
        return self.dequantize(codes, rep(scale), rep(zero), zero_meta, 1, zero_bits)

    def gemm(self, x16, codes, scale, zero, zero_meta, n, k, g, zero_bits):
        """The linear layer of a quantized weight [SK "HQQLinear layer": the layer computes with
        the dequantized weight]: Y = X · W_r^T, W_r the binary16 reconstruction of the axis-1
        quantized [n, k] weight (this oracle's dequantize), X binary16 [m, k]. Products of
        binary16 values are exact in binary64; the sums are binary64 (numpy matmul)."""
        w = self.dequantize(codes, scale, zero, zero_meta, g, zero_bits)
        w = w.view(np.float16).astype(np.float64).reshape(n, k)
        x = np.ascontiguousarray(x16, np.uint16).view(np.float16).astype(np.float64)
        return x.reshape(-1, k) @ w.T

    def packed_bytes(self, n, nbits) -> int:
        return int(self.L.hqo_packed_bytes(n, nbits))

    def pack(self, codes, nbits):
        codes = np.ascontiguousarray(codes, np.uint8).reshape(-1)
        out = np.empty(self.packed_bytes(codes.size, nbits), np.uint8)
        self.L.hqo_pack(codes, codes.size, nbits, out)
        return out

    def unpack(self, packed, n, nbits):
        packed = np.ascontiguousarray(packed, np.uint8).reshape(-1)
        assert packed.size >= self.packed_bytes(n, nbits)
        codes = np.empty(n, np.uint8)
        self.L.hqo_unpack(packed, n, nbits, codes)
        return codes

    def dequantize(self, codes, scale, zero, zero_meta, g, zero_bits):
        codes = np.ascontiguousarray(codes, np.uint8).reshape(-1)
        scale = np.ascontiguousarray(scale, np.uint16)
        zero = np.ascontiguousarray(zero, np.uint16 if zero_bits == 16 else np.uint8)
        meta = None if zero_meta is None else np.ascontiguousarray(zero_meta, np.uint16)
        out = np.empty(codes.size, np.uint16)
        self.L.hqo_dequantize(codes, scale, _ptr(zero), _ptr(meta), codes.size, g, zero_bits,
                              out)
        return out

    def mse(self, w16, codes, scale, zero, zero_meta, g, zero_bits) -> float:
        w16 = np.ascontiguousarray(w16, np.uint16).reshape(-1)
        codes = np.ascontiguousarray(codes, np.uint8).reshape(-1)
        scale = np.ascontiguousarray(scale, np.uint16)
        zero = np.ascontiguousarray(zero, np.uint16 if zero_bits == 16 else np.uint8)
        meta = None if zero_meta is None else np.ascontiguousarray(zero_meta, np.uint16)
        return float(self.L.hqo_mse(w16, codes, scale, _ptr(zero), _ptr(meta), w16.size, g,
                                    zero_bits))
