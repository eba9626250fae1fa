"""The C ABI library on the host: it loads, exports what include/hqq.h declares, and rejects
invalid arguments before any HIP call (so these run without a GPU)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def H():
    from calibration_free_weight_amd import hqq
    if not os.path.exists(hqq.LIB_PATH):
        from calibration_free_weight_amd import build
        build.build()
    return hqq


def declared_functions():
    src = open(os.path.join(ROOT, "include", "hqq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hqq_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(H):
    names = declared_functions()
    assert len(names) >= 9
    L = H.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(H.EXPORTS) == names


def test_packed_bytes(H):
    f = H.hqq_packed_bytes
    assert f(0, 4) == 0 and f(1, 4) == 1 and f(2, 4) == 1 and f(3, 4) == 2
    assert f(16, 2) == 4 and f(17, 2) == 5 and f(8, 1) == 1 and f(9, 1) == 2
    assert f(10, 3) == 4 and f(11, 3) == 8 and f(1, 3) == 4 and f(5, 8) == 5
    assert f(10, 5) == 0


def _job(H, **kw):
    base = dict(W=0x1000, rows=64, cols=256, nbits=4, group_size=64, axis=1, p=0.7, beta=1.0,
                kappa=1.01, iters=20, early_stop=1, zero_bits=8, packed=0x2000, scale=0x3000,
                zero=0x4000, zero_meta=0x5000, passes=None)
    base.update(kw)
    return H.hqq_job(**base)


BAD = [
    (dict(nbits=5), 1), (dict(nbits=0), 1), (dict(axis=0, rows=72), 1), (dict(axis=2), 1),
    (dict(group_size=48), 1), (dict(group_size=0), 1), (dict(group_size=8, cols=256), 2),
    (dict(p=0.0), 1), (dict(p=1.5), 1), (dict(p=float("nan")), 1), (dict(beta=0.0), 1),
    (dict(kappa=-1.0), 1), (dict(iters=-1), 1), (dict(iters=255), 1), (dict(early_stop=2), 1),
    (dict(zero_bits=4), 1), (dict(W=None), 1), (dict(zero_meta=None), 1),
    (dict(W=0x1002), 1), (dict(packed=0x2008), 1), (dict(rows=-1), 1),
    (dict(rows=1 << 20, cols=1 << 18, group_size=64), 1),    # 2^32 groups
]


@pytest.mark.parametrize("kw,status", BAD, ids=[str(b[0]) for b in BAD])
def test_invalid_arguments_rejected(H, kw, status):
    L = H.lib()
    j = _job(H, **kw)
    st = L.hqq_quantize_batch(C.byref(j), 1, None, 0, None)
    assert st == status
    assert L.hqq_last_error().decode() != ""
    assert H.hqq_status_string(st) != "unknown status"
    arr = (H.hqq_job * 1)(j)
    assert L.hqq_workspace_bytes(arr, 1) == 2 ** 64 - 1
    assert L.hqq_batch_check(C.byref(j), 1, None, 0, None) == status


def test_workspace_sizing_and_check(H):
    L = H.lib()
    j8 = _job(H)
    arr = (H.hqq_job * 1)(j8)
    need = L.hqq_workspace_bytes(arr, 1)
    ng = 64 * 256 // 64
    assert need >= 4 * ng and need % 256 == 0
    assert L.hqq_quantize_batch(C.byref(j8), 1, None, 0, None) == H.HQQ_ERR_WORKSPACE
    assert L.hqq_quantize_batch(C.byref(j8), 1, C.c_void_p(0x100000), need - 1, None) == \
        H.HQQ_ERR_WORKSPACE
    assert L.hqq_quantize_batch(C.byref(j8), 1, C.c_void_p(0x100010), need, None) == \
        H.HQQ_ERR_ARG                                   # misaligned workspace
    j16 = _job(H, zero_bits=16, zero_meta=None)
    n16 = L.hqq_workspace_bytes((H.hqq_job * 1)(j16), 1)
    assert 0 < n16 < need and n16 % 256 == 0
    assert L.hqq_quantize_batch(C.byref(j16), 1, None, 0, None) == H.HQQ_ERR_WORKSPACE
    # two jobs of one class need one table of two entries, not two workspaces
    two = (H.hqq_job * 2)(j16, j16)
    assert L.hqq_workspace_bytes(two, 2) < 2 * n16 + 512
    # empty tensors are valid and need nothing
    je = _job(H, rows=0, W=None, packed=None, scale=None, zero=None, zero_meta=None)
    assert L.hqq_workspace_bytes((H.hqq_job * 1)(je), 1) == 0
    assert L.hqq_quantize_batch(C.byref(je), 1, None, 0, None) == H.HQQ_OK


def test_other_entry_points_validate(H):
    L = H.lib()
    assert L.hqq_pack(None, 10, 4, None, None) == H.HQQ_ERR_ARG
    assert L.hqq_pack(C.c_void_p(0x1000), 10, 6, C.c_void_p(0x2000), None) == H.HQQ_ERR_ARG
    assert L.hqq_pack(C.c_void_p(0x1000), 0, 4, None, None) == H.HQQ_OK
    assert L.hqq_unpack(C.c_void_p(0x1001), 10, 3, C.c_void_p(0x2000), None) == H.HQQ_ERR_ARG
    assert L.hqq_dequantize(C.c_void_p(0x1000), C.c_void_p(0x2000), C.c_void_p(0x3000), None,
                            4, 64, 4, 64, 1, 8, C.c_void_p(0x4000), None) == H.HQQ_ERR_ARG
    # axis 0 needs group_size to divide rows; then the null buffers are the error
    assert L.hqq_dequantize(None, None, None, None, 4, 64, 4, 64, 0, 16, None, None) == \
        H.HQQ_ERR_ARG
    assert "divide rows" in L.hqq_last_error().decode()
    assert L.hqq_dequantize(None, None, None, None, 128, 3, 4, 64, 0, 16, None, None) == \
        H.HQQ_ERR_ARG
    assert "non-null" in L.hqq_last_error().decode()
    assert L.hqq_dequantize(None, None, None, None, 128, 3, 4, 8, 0, 16, None, None) == \
        H.HQQ_ERR_UNSUPPORTED


def test_scale_entry_points_validate(H):
    L = H.lib()
    s, q, m, o = (C.c_void_p(a) for a in (0x1000, 0x2000, 0x3000, 0x4000))
    ok, arg = H.HQQ_OK, H.HQQ_ERR_ARG
    for g in (7, 4, 1024, 96, 0, -128):                       # not a power of two in [8, 512]
        assert L.hqq_requant_scales(s, 100, g, q, m, None) == arg
        assert L.hqq_dequantize_scales(q, m, 100, g, o, None) == arg
    assert L.hqq_requant_scales(s, -1, 128, q, m, None) == arg
    assert L.hqq_requant_scales(s, 0, 128, None, None, None) == ok       # empty: nothing to do
    assert L.hqq_dequantize_scales(None, None, 0, 128, None, None) == ok
    assert L.hqq_requant_scales(None, 100, 128, q, m, None) == arg
    assert L.hqq_requant_scales(s, 100, 128, q, None, None) == arg
    assert L.hqq_requant_scales(C.c_void_p(0x1008), 100, 128, q, m, None) == arg   # scale 16 B
    assert L.hqq_requant_scales(s, 100, 128, C.c_void_p(0x2004), m, None) == arg   # scale_q 8 B
    assert L.hqq_requant_scales(s, 100, 128, q, C.c_void_p(0x3002), None) == arg   # meta 4 B
    assert L.hqq_dequantize_scales(q, m, 100, 128, C.c_void_p(0x4008), None) == arg
    assert L.hqq_dequantize_scales(q, m, 100, 128, None, None) == arg
    assert "scale_group" in L.hqq_last_error().decode() or L.hqq_last_error().decode() != ""


def test_streamed_entry_points_validate(H):
    L = H.lib()
    j = _job(H, rows=64, cols=256)                       # 32 KiB of binary16 weights
    arr = (H.hqq_job * 2)(j, _job(H, rows=128, cols=256, W=0x9000))
    big = 1 << 20
    assert L.hqq_streamed_workspace_bytes(arr, 2, big) not in (0, 2 ** 64 - 1)
    assert L.hqq_streamed_workspace_bytes(arr, 2, 2 * 32768) == 2 ** 64 - 1   # 64 KiB tensor
    st = L.hqq_quantize_streamed(arr, 2, C.c_void_p(0x100000), 2 * 32768, None, 0, None, None)
    assert st == H.HQQ_ERR_WORKSPACE and "half the staging" in L.hqq_last_error().decode()
    st = L.hqq_quantize_streamed(arr, 2, None, big, C.c_void_p(0x200000), big, None, None)
    assert st == H.HQQ_ERR_ARG and "staging" in L.hqq_last_error().decode()
    st = L.hqq_quantize_streamed(arr, 2, C.c_void_p(0x100010), big, C.c_void_p(0x200000), big,
                                 None, None)
    assert st == H.HQQ_ERR_ARG                            # staging not 256-byte aligned
    st = L.hqq_quantize_streamed(arr, 2, C.c_void_p(0x100000), big, None, 0, None, None)
    assert st == H.HQQ_ERR_WORKSPACE
    bad = (H.hqq_job * 1)(_job(H, nbits=5))
    assert L.hqq_quantize_streamed(bad, 1, C.c_void_p(0x100000), big, None, 0, None, None) == \
        H.HQQ_ERR_ARG
    empty = (H.hqq_job * 1)(_job(H, rows=0))
    assert L.hqq_quantize_streamed(empty, 1, None, 0, None, 0, None, None) == H.HQQ_OK


def test_gemm_f16_validates(H):
    """hqq_gemm_f16 rejects bad sizes and alignments on the host (fake device addresses: a
    rejected call reaches no HIP call) and treats empty products as done."""
    L = H.lib()
    X, W, Y = (C.c_void_p(a) for a in (0x1000, 0x2000, 0x3000))
    ok, arg = H.HQQ_OK, H.HQQ_ERR_ARG
    g = lambda x, m, w, n, k, y: L.hqq_gemm_f16(x, m, w, n, k, y, None)
    assert g(None, 0, None, 64, 128, None) == ok                      # M = 0
    assert g(None, 4, None, 0, 128, None) == ok                       # N = 0
    assert g(X, -1, W, 64, 128, Y) == arg
    assert g(X, 4, W, 64, -8, Y) == arg
    for k in (0, 4, 100, (1 << 22) + 8):                              # K % 8, 0 < K <= 2^22
        assert g(X, 4, W, 64, k, Y) == arg, k
    assert g(None, 4, W, 64, 128, Y) == arg
    assert g(X, 4, None, 64, 128, Y) == arg
    assert g(X, 4, W, 64, 128, None) == arg
    assert g(C.c_void_p(0x1008), 4, W, 64, 128, Y) == arg              # X 16-byte aligned
    assert g(X, 4, C.c_void_p(0x2008), 64, 128, Y) == arg              # Wr 16-byte aligned
    assert g(X, 4, W, 64, 128, C.c_void_p(0x3001)) == arg              # Y 2-byte aligned
    assert g(X, 1 << 30, W, 64, 4096, Y) == arg                        # M*K too large


def test_gemm_validates(H):
    L = H.lib()
    p = [C.c_void_p(a) for a in (0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000)]
    X, P, S, Z, M_, Y = p
    ok, arg, uns = H.HQQ_OK, H.HQQ_ERR_ARG, H.HQQ_ERR_UNSUPPORTED

    def gm(*a, ws=None, wb=0):                   # no workspace unless given, default stream
        return L.hqq_gemm(*a, ws, wb, None)
    assert gm(X, 0, None, None, None, None, 64, 128, 4, 64, 16, None) == ok
    assert gm(X, -1, P, S, Z, None, 64, 128, 4, 64, 16, Y) == arg
    assert gm(X, 4, P, S, Z, None, 64, 100, 4, 64, 16, Y) == arg      # g | K
    assert gm(X, 4, P, S, Z, None, 64, 128, 5, 64, 16, Y) == arg
    assert gm(X, 4, P, S, Z, None, 64, 128, 4, 8, 16, Y) == uns
    assert gm(X, 4, P, S, Z, None, 64, 128, 4, 64, 12, Y) == arg
    assert gm(X, 4, P, S, Z, None, 64, 128, 4, 64, 8, Y) == arg       # no meta
    assert gm(None, 4, P, S, Z, None, 64, 128, 4, 64, 16, Y) == arg
    assert gm(C.c_void_p(0x1008), 4, P, S, Z, None, 64, 128, 4, 64, 16, Y) == arg
    assert gm(X, 4, C.c_void_p(0x2002), S, Z, None, 64, 130, 3, 10, 16, Y) != ok
    # the optional workspace of the reconstruct-once path (M > 64)
    need = L.hqq_gemm_workspace_bytes(65, 64, 128)
    assert need == 64 * 128 * 2 and L.hqq_gemm_workspace_bytes(64, 64, 128) == 0
    assert L.hqq_gemm_workspace_bytes(100, 11008, 4096) == 11008 * 4096 * 2
    assert L.hqq_gemm_workspace_bytes(100, 3, 16) == 256                 # rounded up
    a = (X, 65, P, S, Z, None, 64, 128, 4, 64, 16, Y)
    assert gm(*a, ws=C.c_void_p(0x7000), wb=need - 1) == H.HQQ_ERR_WORKSPACE
    assert gm(*a, ws=C.c_void_p(0x7008), wb=need) == arg                # 16-byte alignment


def test_noalloc_rejects_before_any_device_call(H):
    """The no-workspace entry point validates like hqq_quantize and refuses a tensor whose
    scratch would exceed its static 64 MiB, both before touching the device."""
    L = H.lib()
    args = [C.c_void_p(0x1000), 64, 256, 5, 64, 1, 0.7, 1.0, 1.01, 20, 1, 8,
            C.c_void_p(0x2000), C.c_void_p(0x3000), C.c_void_p(0x4000), C.c_void_p(0x5000),
            None, None]
    assert L.hqq_quantize_noalloc(*args) == 1                      # nbits = 5
    big = list(args)
    big[1], big[2], big[3], big[5], big[11] = 8192, 8192, 4, 0, 16  # axis 0: ~156 MiB of scratch
    assert L.hqq_quantize_noalloc(*big) == 3
    assert "static scratch" in L.hqq_last_error().decode()


def test_gemm_multi_validates(H):
    """hqq_gemm_multi checks every weight before launching anything (fake device addresses:
    a rejected call reaches no HIP call); errors name the weight; empty work is done."""
    L = H.lib()
    X, P, S, Z, Y, WS = (C.c_void_p(a) for a in (0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x8000))
    ok, arg, uns, wsz = H.HQQ_OK, H.HQQ_ERR_ARG, H.HQQ_ERR_UNSUPPORTED, H.HQQ_ERR_WORKSPACE

    def w(N=64, nbits=4, g=64, zb=16, meta=None, y=Y, packed=P):
        return H.hqq_gemm_weight(packed, S, Z, meta, N, nbits, g, zb, y)

    def gm(M, K, ws, n=None, work=None, wb=0):
        arr = (H.hqq_gemm_weight * max(len(ws), 1))(*ws)
        return L.hqq_gemm_multi(X, M, K, arr, len(ws) if n is None else n, work, wb, None)
    assert gm(4, 128, []) == ok                                   # no weights
    assert gm(0, 128, [w(), w(N=128)]) == ok                      # M = 0
    assert gm(4, 128, [w(N=0)]) == ok                             # an empty weight
    assert gm(-1, 128, [w()]) == arg
    assert gm(4, 128, [w()], n=-1) == arg
    assert L.hqq_gemm_multi(X, 4, 128, None, 2, None, 0, None) == arg
    assert gm(4, 128, [w(), w(nbits=5)]) == arg
    assert "weight 1" in H.hqq_last_error()
    assert gm(4, 128, [w(g=8)]) == uns
    assert gm(4, 100, [w()]) == arg                               # g | K
    assert gm(4, 128, [w(), w(zb=12)]) == arg
    assert gm(4, 128, [w(zb=8)]) == arg                           # 8-bit zeros need the meta
    assert gm(4, 128, [w(), w(y=None)]) == arg
    assert gm(4, 128, [w(y=C.c_void_p(0x5001))]) == arg           # Y 2-byte aligned
    assert gm(4, 130, [w(nbits=3, g=10, packed=C.c_void_p(0x2002))]) != ok
    big = L.hqq_gemm_workspace_bytes(100, 256, 128)
    assert gm(100, 128, [w(N=64), w(N=256)], work=WS, wb=big - 1) == wsz   # the largest need
    assert gm(100, 128, [w()], work=C.c_void_p(0x8008), wb=big) == arg     # 16-byte aligned
    assert gm(1 << 30, 4096, [w()]) == arg                        # M*K too large
