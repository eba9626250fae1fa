"""Python binding of libhqq: the C ABI of include/hqq.h, argument marshalling only.

Every compute step runs in the HIP library; this module passes device pointers
(``tensor.data_ptr()``), sizes and the current HIP stream through ctypes. PyTorch provides
device memory and streams. There is no fallback: if the library is missing the import of a
function raises.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libhqq.so")

HQQ_OK, HQQ_ERR_ARG, HQQ_ERR_UNSUPPORTED, HQQ_ERR_WORKSPACE, HQQ_ERR_DEVICE = range(5)

# Functions declared in include/hqq.h (checked by the tests against the header).
EXPORTS = ("hqq_packed_bytes", "hqq_workspace_bytes", "hqq_quantize", "hqq_quantize_batch",
           "hqq_solve_batch", "hqq_requant_batch", "hqq_quantize_streamed",
           "hqq_streamed_workspace_bytes", "hqq_dequantize", "hqq_gemm",
           "hqq_gemm_workspace_bytes", "hqq_gemm_f16", "hqq_requant_scales",
           "hqq_dequantize_scales", "hqq_pack", "hqq_unpack", "hqq_status_string",
           "hqq_last_error", "hqq_batch_check", "hqq_debug_solver", "hqq_quantize_noalloc",
           "hqq_gemm_multi")


class HQQError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class hqq_job(C.Structure):
    _fields_ = [("W", C.c_void_p), ("rows", C.c_int64), ("cols", C.c_int64),
                ("nbits", C.c_int), ("group_size", C.c_int), ("axis", C.c_int),
                ("p", C.c_float), ("beta", C.c_float), ("kappa", C.c_float),
                ("iters", C.c_int), ("early_stop", C.c_int), ("zero_bits", C.c_int),
                ("packed", C.c_void_p), ("scale", C.c_void_p), ("zero", C.c_void_p),
                ("zero_meta", C.c_void_p), ("passes", C.c_void_p)]


class hqq_gemm_weight(C.Structure):
    _fields_ = [("packed", C.c_void_p), ("scale", C.c_void_p), ("zero", C.c_void_p),
                ("zero_meta", C.c_void_p), ("N", C.c_int64), ("nbits", C.c_int),
                ("group_size", C.c_int), ("zero_bits", C.c_int), ("Y", C.c_void_p)]


_L = None


def lib():
    """The loaded library. Raises if it has not been built (no CPU fallback exists)."""
    global _L
    if _L is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        vp, i64, i32, f32 = C.c_void_p, C.c_int64, C.c_int, C.c_float
        L.hqq_packed_bytes.restype = C.c_size_t
        L.hqq_packed_bytes.argtypes = [i64, i32]
        L.hqq_workspace_bytes.restype = C.c_size_t
        L.hqq_workspace_bytes.argtypes = [C.POINTER(hqq_job), i32]
        L.hqq_quantize.restype = i32
        L.hqq_quantize.argtypes = [vp, i64, i64, i32, i32, i32, f32, f32, f32, i32, i32, i32,
                                   vp, vp, vp, vp, vp, vp, C.c_size_t, vp]
        L.hqq_quantize_noalloc.restype = i32
        L.hqq_quantize_noalloc.argtypes = [vp, i64, i64, i32, i32, i32, f32, f32, f32, i32, i32,
                                           i32, vp, vp, vp, vp, vp, vp]
        for name in ("hqq_quantize_batch", "hqq_solve_batch", "hqq_requant_batch"):
            getattr(L, name).restype = i32
            getattr(L, name).argtypes = [C.POINTER(hqq_job), i32, vp, C.c_size_t, vp]
        L.hqq_batch_check.restype = i32
        L.hqq_batch_check.argtypes = [C.POINTER(hqq_job), i32, vp, C.c_size_t, vp]
        L.hqq_debug_solver.restype = None
        L.hqq_debug_solver.argtypes = [i64, i32]
        L.hqq_quantize_streamed.restype = i32
        L.hqq_quantize_streamed.argtypes = [C.POINTER(hqq_job), i32, vp, C.c_size_t, vp,
                                            C.c_size_t, vp, vp]
        L.hqq_streamed_workspace_bytes.restype = C.c_size_t
        L.hqq_streamed_workspace_bytes.argtypes = [C.POINTER(hqq_job), i32, C.c_size_t]
        L.hqq_dequantize.restype = i32
        L.hqq_dequantize.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, vp, vp]
        L.hqq_gemm.restype = i32
        L.hqq_gemm.argtypes = [vp, i64, vp, vp, vp, vp, i64, i64, i32, i32, i32, vp, vp,
                               C.c_size_t, vp]
        L.hqq_gemm_workspace_bytes.restype = C.c_size_t
        L.hqq_gemm_workspace_bytes.argtypes = [i64, i64, i64]
        L.hqq_gemm_multi.restype = i32
        L.hqq_gemm_multi.argtypes = [vp, i64, i64, C.POINTER(hqq_gemm_weight), i32, vp, C.c_size_t, vp]
        L.hqq_gemm_f16.restype = i32
        L.hqq_gemm_f16.argtypes = [vp, i64, vp, i64, i64, vp, vp]
        L.hqq_requant_scales.restype = i32
        L.hqq_requant_scales.argtypes = [vp, i64, i32, vp, vp, vp]
        L.hqq_dequantize_scales.restype = i32
        L.hqq_dequantize_scales.argtypes = [vp, vp, i64, i32, vp, vp]
        L.hqq_pack.restype = i32
        L.hqq_pack.argtypes = [vp, i64, i32, vp, vp]
        L.hqq_unpack.restype = i32
        L.hqq_unpack.argtypes = [vp, i64, i32, vp, vp]
        L.hqq_status_string.restype = C.c_char_p
        L.hqq_status_string.argtypes = [i32]
        L.hqq_last_error.restype = C.c_char_p
        L.hqq_last_error.argtypes = []
        _L = L
    return _L


def _p(t):
    """Device pointer of a tensor (or None)."""
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return C.c_void_p(int(stream))
    import torch
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(st: int):
    if st != HQQ_OK:
        L = lib()
        raise HQQError(st, f"{L.hqq_status_string(st).decode()}: {L.hqq_last_error().decode()}")


def hqq_status_string(status: int) -> str:
    return lib().hqq_status_string(status).decode()


def hqq_last_error() -> str:
    return lib().hqq_last_error().decode()


def hqq_packed_bytes(n_codes: int, nbits: int) -> int:
    return int(lib().hqq_packed_bytes(n_codes, nbits))


def make_job(W, nbits, group_size, axis, p, beta, kappa, iters, early_stop, zero_bits,
             packed, scale, zero, zero_meta, passes=None) -> hqq_job:
    rows, cols = W.shape
    return hqq_job(_p(W), rows, cols, nbits, group_size, axis, p, beta, kappa, iters,
                   int(early_stop), zero_bits, _p(packed), _p(scale), _p(zero),
                   _p(zero_meta), _p(passes))


def hqq_workspace_bytes(jobs) -> int:
    arr = (hqq_job * len(jobs))(*jobs)
    n = int(lib().hqq_workspace_bytes(arr, len(jobs)))
    if n == (1 << 64) - 1:
        raise HQQError(HQQ_ERR_ARG, "invalid job in workspace query")
    return n


def hqq_quantize(W, nbits, group_size, axis, p, beta, kappa, iters, early_stop, zero_bits,
                 packed, scale, zero, zero_meta, passes, workspace, stream=None) -> None:
    rows, cols = W.shape
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().hqq_quantize(_p(W), rows, cols, nbits, group_size, axis, p, beta, kappa,
                              iters, int(early_stop), zero_bits, _p(packed), _p(scale),
                              _p(zero), _p(zero_meta), _p(passes), _p(workspace), wsb,
                              _stream(stream)))


def hqq_quantize_noalloc(W, nbits, group_size, axis, p, beta, kappa, iters, early_stop,
                         zero_bits, packed, scale, zero, zero_meta, passes, stream=None) -> None:
    """hqq_quantize on the library's static scratch (no workspace argument)."""
    rows, cols = W.shape
    _check(lib().hqq_quantize_noalloc(_p(W), rows, cols, nbits, group_size, axis, p, beta,
                                      kappa, iters, int(early_stop), zero_bits, _p(packed),
                                      _p(scale), _p(zero), _p(zero_meta), _p(passes),
                                      _stream(stream)))


def _batch(fn, jobs, workspace, stream):
    arr = (hqq_job * len(jobs))(*jobs)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(fn(arr, len(jobs), _p(workspace), wsb, _stream(stream)))


def hqq_quantize_batch(jobs, workspace, stream=None) -> None:
    _batch(lib().hqq_quantize_batch, jobs, workspace, stream)


def hqq_solve_batch(jobs, workspace, stream=None) -> None:
    _batch(lib().hqq_solve_batch, jobs, workspace, stream)


def hqq_requant_batch(jobs, workspace, stream=None) -> None:
    _batch(lib().hqq_requant_batch, jobs, workspace, stream)


def hqq_batch_check(jobs, workspace, stream=None) -> None:
    """Waits for `stream`; raises HQQError (HQQ_ERR_DEVICE) if the last solve on this
    workspace left groups unwritten."""
    _batch(lib().hqq_batch_check, jobs, workspace, stream)


def hqq_debug_solver(step_budget: int = 0, pass_layout: int = 0) -> None:
    """Test hook: a fixed solver step budget (0 = default) and the solver kernel (0 = by
    size, 1 = persistent with one lane per group, 2 = persistent with several lanes per
    group, 3 = lockstep)."""
    lib().hqq_debug_solver(int(step_budget), int(pass_layout))


def hqq_streamed_workspace_bytes(jobs, staging_bytes) -> int:
    arr = (hqq_job * len(jobs))(*jobs)
    n = int(lib().hqq_streamed_workspace_bytes(arr, len(jobs), staging_bytes))
    if n == (1 << 64) - 1:
        raise HQQError(HQQ_ERR_ARG, "invalid job, or a tensor larger than half the staging")
    return n


def hqq_quantize_streamed(jobs, staging, workspace, stream=None, copy_stream=None) -> None:
    """jobs[i].W are host pointers (pinned); staging and workspace are device tensors."""
    arr = (hqq_job * len(jobs))(*jobs)
    sb = staging.numel() * staging.element_size()
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    cs = _stream(copy_stream) if copy_stream is not None else _stream(stream)
    _check(lib().hqq_quantize_streamed(arr, len(jobs), _p(staging), sb, _p(workspace), wsb,
                                       _stream(stream), cs))


def hqq_dequantize(packed, scale, zero, zero_meta, rows, cols, nbits, group_size, axis,
                   zero_bits, W_out, stream=None) -> None:
    _check(lib().hqq_dequantize(_p(packed), _p(scale), _p(zero), _p(zero_meta), rows, cols,
                                nbits, group_size, axis, zero_bits, _p(W_out),
                                _stream(stream)))


def hqq_gemm(X, packed, scale, zero, zero_meta, N, K, nbits, group_size, zero_bits, Y,
             workspace=None, stream=None) -> None:
    """Y[M, N] = X[M, K] . W_r^T for a packed axis-1 quantized weight [N, K]; `workspace`
    (optional, at least hqq_gemm_workspace_bytes(M, N, K) bytes) selects the reconstruct-once
    path for M > 64."""
    M = X.shape[0]
    wb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().hqq_gemm(_p(X), M, _p(packed), _p(scale), _p(zero), _p(zero_meta), N, K,
                          nbits, group_size, zero_bits, _p(Y), _p(workspace), wb,
                          _stream(stream)))


def hqq_gemm_multi(X, weights, workspace=None, stream=None) -> None:
    """Several weights [N_i, K] multiplied by the same X: `weights` is a list of dicts with
    packed, scale, zero, zero_meta, N, nbits, group_size, zero_bits and Y (as hqq_gemm's
    arguments); each Y_i gets what hqq_gemm would write."""
    M, K = X.shape
    arr = (hqq_gemm_weight * max(len(weights), 1))()
    for i, w in enumerate(weights):
        arr[i] = hqq_gemm_weight(_p(w["packed"]), _p(w["scale"]), _p(w["zero"]),
                                 _p(w.get("zero_meta")), w["N"], w["nbits"], w["group_size"],
                                 w["zero_bits"], _p(w["Y"]))
    wb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().hqq_gemm_multi(_p(X), M, K, arr, len(weights), _p(workspace), wb,
                                _stream(stream)))


def hqq_gemm_workspace_bytes(M, N, K) -> int:
    return int(lib().hqq_gemm_workspace_bytes(M, N, K))


def hqq_gemm_f16(X, Wr, N, K, Y, stream=None) -> None:
    """Y[M, N] = X[M, K] . Wr^T for a binary16 weight Wr [N, K] (as hqq_dequantize writes it)."""
    _check(lib().hqq_gemm_f16(_p(X), X.shape[0], _p(Wr), N, K, _p(Y), _stream(stream)))


def hqq_requant_scales(scale, n, scale_group, scale_q, scale_meta, stream=None) -> None:
    _check(lib().hqq_requant_scales(_p(scale), n, scale_group, _p(scale_q), _p(scale_meta),
                                    _stream(stream)))


def hqq_dequantize_scales(scale_q, scale_meta, n, scale_group, scale_out, stream=None) -> None:
    _check(lib().hqq_dequantize_scales(_p(scale_q), _p(scale_meta), n, scale_group,
                                       _p(scale_out), _stream(stream)))


def requant_scales(scale, scale_group=128, stream=None):
    """Allocate and fill 8-bit scales for a binary16 scale tensor: (scale_q, scale_meta)."""
    import torch
    n = scale.numel()
    sq = torch.empty(max(n, 1), dtype=torch.uint8, device=scale.device)
    meta = torch.empty(max(2 * ((n + scale_group - 1) // scale_group), 2), dtype=torch.float16,
                       device=scale.device)
    hqq_requant_scales(scale, n, scale_group, sq, meta, stream)
    return sq[:n], meta[:2 * ((n + scale_group - 1) // scale_group)]


def hqq_pack(codes, n_codes, nbits, packed, stream=None) -> None:
    _check(lib().hqq_pack(_p(codes), n_codes, nbits, _p(packed), _stream(stream)))


def hqq_unpack(packed, n_codes, nbits, codes, stream=None) -> None:
    _check(lib().hqq_unpack(_p(packed), n_codes, nbits, _p(codes), _stream(stream)))


# ---- allocation helpers (PyTorch device memory for the outputs) -----------------------------
def alloc_outputs(rows, cols, nbits, group_size, zero_bits, device, passes=False):
    """Output tensors of one job: packed (uint8, 16-byte aligned by the allocator), scale,
    zero, zero_meta (or None) and passes (or None)."""
    import torch
    ng = rows * cols // group_size
    out = dict(
        packed=torch.empty(max(hqq_packed_bytes(rows * cols, nbits), 1), dtype=torch.uint8,
                           device=device),
        scale=torch.empty(ng, dtype=torch.float16, device=device),
        zero=torch.empty(ng, dtype=torch.float16 if zero_bits == 16 else torch.uint8,
                         device=device),
        zero_meta=torch.empty(2, dtype=torch.float16, device=device) if zero_bits == 8 else None,
        passes=torch.empty(ng, dtype=torch.uint8, device=device) if passes else None,
    )
    return out


def alloc_workspace(jobs, device):
    import torch
    n = hqq_workspace_bytes(jobs)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device) if n > 0 else None


def quantize(W, nbits, group_size, axis=1, p=0.7, beta=1.0, kappa=1.01, iters=20,
             early_stop=True, zero_bits=16, passes=False, stream=None):
    """Allocate outputs and a workspace, then call hqq_quantize. Returns the output dict."""
    rows, cols = W.shape
    out = alloc_outputs(rows, cols, nbits, group_size, zero_bits, W.device, passes)
    job = make_job(W, nbits, group_size, axis, p, beta, kappa, iters, early_stop, zero_bits,
                   out["packed"], out["scale"], out["zero"], out["zero_meta"], out["passes"])
    ws = alloc_workspace([job], W.device)
    hqq_quantize(W, nbits, group_size, axis, p, beta, kappa, iters, early_stop, zero_bits,
                 out["packed"], out["scale"], out["zero"], out["zero_meta"], out["passes"],
                 ws, stream)
    out["workspace"] = ws
    out["job"] = job
    return out
