"""Host-side checks of the C ABI: the library loads, exports every declared entry
point, and rejects bad arguments before launching anything (no GPU needed)."""
import os
import re
import subprocess

import pytest

import bit_mixed_precision_tri_amd as tri

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tri.h")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tri_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared()
    assert {"tri_row_bytes", "tri_pack2", "tri_pack16", "tri_unpack", "tri_linear"} <= set(names)
    out = subprocess.check_output(["nm", "-D", "--defined-only", tri.LIB_PATH], text=True)
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    L = tri.lib()
    for n in names:
        assert getattr(L, n) is not None


def test_row_bytes():
    assert tri.tri_row_bytes(4096, tri.TRI_FMT_2BIT) == 1024
    assert tri.tri_row_bytes(11008, tri.TRI_FMT_2BIT) == 2752
    assert tri.tri_row_bytes(4096, tri.TRI_FMT_1P6BIT) == 832
    assert tri.tri_row_bytes(11008, tri.TRI_FMT_1P6BIT) == 2208
    assert tri.tri_row_bytes(1, tri.TRI_FMT_2BIT) == 16 and tri.tri_row_bytes(81, tri.TRI_FMT_1P6BIT) == 32
    assert tri.tri_row_bytes(0, tri.TRI_FMT_2BIT) == -1
    assert tri.tri_row_bytes(10, 5) == -1


def test_status_strings():
    for code in (0, -1, -2, -3, 7):
        assert isinstance(tri.tri_status_string(code), str) and tri.tri_status_string(code)


def test_select_algo():
    F2, F16 = tri.TRI_FMT_2BIT, tri.TRI_FMT_1P6BIT
    assert tri.tri_select_algo(1, 4096, 4096, F2) == tri.TRI_ALGO_SMALLM   # the MFMA kernel also serves M = 1
    assert tri.tri_select_algo(1, 4096, 4096, F16) == tri.TRI_ALGO_SMALLM
    assert tri.tri_select_algo(16, 4096, 4096, F2) == tri.TRI_ALGO_SMALLM
    # above 16 rows, the cheaper of the two by the fitted cost model; each pair brackets a crossover measured on
    # MI355X, on points where the faster of the two won by at least 15%
    S, G = tri.TRI_ALGO_SMALLM, tri.TRI_ALGO_GEMM
    for M, N, K, f, want in [
            (17, 4096, 4096, F2, S), (128, 4096, 4096, F2, S), (384, 4096, 4096, F2, G),
            (128, 4096, 4096, F16, S), (256, 4096, 4096, F16, G),
            (48, 11008, 4096, F2, S), (96, 11008, 4096, F2, G),          # 64-row GEMM tiles at a middling M
            (32, 11008, 4096, F16, S), (96, 11008, 4096, F16, G),
            (128, 4096, 11008, F2, S), (192, 4096, 11008, F2, G),
            (128, 4096, 11008, F16, S), (256, 4096, 11008, F16, G),
            (17, 28672, 8192, F2, G), (17, 28672, 8192, F16, G),
            (32, 8192, 28672, F2, S), (64, 8192, 28672, F2, G),          # rows past eight steps per wave
            (48, 8192, 28672, F16, S), (96, 8192, 28672, F16, G),
            (2048, 28672, 8192, F2, G), (2048, 8192, 28672, F16, G)]:
        assert tri.tri_select_algo(M, N, K, f) == want, (M, N, K, f)
    assert tri.tri_select_algo(0, 4096, 4096, F2) == tri.TRI_EINVAL
    assert tri.tri_select_algo(1, 4096, 4096, 3) == tri.TRI_EINVAL


# fake device addresses: these calls must fail validation, so nothing is dereferenced or launched
A, B, C, ODD = 4096, 8192, 12288, 4097


def raw(name, *args):
    return getattr(tri.lib(), name)(*args)


def test_linear_argument_errors_launch_nothing():
    F2 = tri.TRI_FMT_2BIT
    s = None
    assert raw("tri_linear", None, B, 1.0, 1, 4, 64, F2, C, s) == tri.TRI_EINVAL
    assert raw("tri_linear", A, None, 1.0, 1, 4, 64, F2, C, s) == tri.TRI_EINVAL
    assert raw("tri_linear", A, B, 1.0, 1, 4, 64, F2, None, s) == tri.TRI_EINVAL
    for (M, N, K) in [(0, 4, 64), (1, 0, 64), (1, 4, 0), (-1, 4, 64), (1, 1 << 31, 64), (1, 4, 1 << 31)]:
        assert raw("tri_linear", A, B, 1.0, M, N, K, F2, C, s) == tri.TRI_EINVAL
    assert raw("tri_linear", A, B, 1.0, 1, 4, 64, 2, C, s) == tri.TRI_EINVAL
    assert raw("tri_linear", ODD, B, 1.0, 1, 4, 64, F2, C, s) == tri.TRI_EALIGN
    assert raw("tri_linear", A, ODD, 1.0, 1, 4, 64, F2, C, s) == tri.TRI_EALIGN
    assert raw("tri_linear", A, B, 1.0, 1, 4, 64, F2, ODD, s) == tri.TRI_EALIGN
    # a kernel family that cannot serve the shape
    assert raw("tri_linear_algo", A, B, 1.0, 2, 4, 64, F2, C, tri.TRI_ALGO_GEMV, s) == tri.TRI_EINVAL
    assert raw("tri_linear_algo", A, B, 1.0, 1, 4, 64, tri.TRI_FMT_1P6BIT, C, tri.TRI_ALGO_GEMV, s) == tri.TRI_EINVAL
    assert raw("tri_linear_algo", A, B, 1.0, 1, 4, 64, F2, C, 9, s) == tri.TRI_EINVAL


def test_pack_argument_errors_launch_nothing():
    s = None
    for name in ("tri_pack2", "tri_pack16"):
        assert raw(name, None, 4, 64, B, s) == tri.TRI_EINVAL
        assert raw(name, A, 4, 64, None, s) == tri.TRI_EINVAL
        assert raw(name, A, 0, 64, B, s) == tri.TRI_EINVAL
        assert raw(name, A, 4, 0, B, s) == tri.TRI_EINVAL
        assert raw(name, A, 4, 64, ODD, s) == tri.TRI_EALIGN
    assert raw("tri_unpack", B, 4, 64, 2, A, s) == tri.TRI_EINVAL
    assert raw("tri_unpack", ODD, 4, 64, 0, A, s) == tri.TRI_EALIGN
    assert raw("tri_unpack", B, 4, 64, 0, None, s) == tri.TRI_EINVAL


def test_probe_argument_errors_launch_nothing():
    assert raw("tri_probe_read", A, 15, B, None) == tri.TRI_EINVAL
    assert raw("tri_probe_read", ODD, 16, B, None) == tri.TRI_EALIGN
    assert raw("tri_probe_copy", A, B, 24, None) == tri.TRI_EINVAL
    assert raw("tri_probe_copy", A, ODD, 32, None) == tri.TRI_EALIGN


def test_binding_raises_on_error_status():
    with pytest.raises(tri.TriError):
        tri.tri_linear(A, B, 1.0, 0, 4, 64, tri.TRI_FMT_2BIT, C, stream=0)


def test_grouped_argument_errors_launch_nothing():
    import ctypes
    F2 = tri.TRI_FMT_2BIT
    s = None
    ptrs = lambda *v: (ctypes.c_void_p * len(v))(*v)
    floats = lambda *v: (ctypes.c_float * len(v))(*v)
    ints = lambda *v: (ctypes.c_int64 * len(v))(*v)
    wp, sc, nn, yy = ptrs(B, B), floats(1.0, 1.0), ints(4, 8), ptrs(C, C)
    for G in (0, -1, tri.TRI_MAX_GROUPS + 1):
        assert raw("tri_linear_grouped", A, wp, sc, 1, nn, 64, F2, yy, G, s) == tri.TRI_EINVAL
    assert raw("tri_linear_grouped", A, None, sc, 1, nn, 64, F2, yy, 2, s) == tri.TRI_EINVAL
    assert raw("tri_linear_grouped", A, wp, None, 1, nn, 64, F2, yy, 2, s) == tri.TRI_EINVAL
    assert raw("tri_linear_grouped", A, wp, sc, 1, None, 64, F2, yy, 2, s) == tri.TRI_EINVAL
    assert raw("tri_linear_grouped", A, wp, sc, 1, nn, 64, F2, None, 2, s) == tri.TRI_EINVAL
    # any bad matrix rejects the whole call
    assert raw("tri_linear_grouped", A, ptrs(B, ODD), sc, 1, nn, 64, F2, yy, 2, s) == tri.TRI_EALIGN
    assert raw("tri_linear_grouped", A, wp, sc, 1, ints(4, 0), 64, F2, yy, 2, s) == tri.TRI_EINVAL
    assert raw("tri_linear_grouped", A, wp, sc, 1, nn, 64, F2, ptrs(C, None), 2, s) == tri.TRI_EINVAL
    assert raw("tri_linear_grouped", None, wp, sc, 1, nn, 64, F2, yy, 2, s) == tri.TRI_EINVAL


def test_quantize_workspace_and_argument_errors_launch_nothing():
    F2 = tri.TRI_FMT_2BIT
    s = None
    assert tri.tri_quantize_workspace_bytes(0, 5) == -1
    assert tri.tri_quantize_workspace_bytes(5, 0) == -1
    assert tri.tri_quantize_workspace_bytes(1, 1) == 8
    assert tri.tri_quantize_workspace_bytes(28672, 8192) == 8 * 2048
    need = tri.tri_quantize_workspace_bytes(4, 64)
    assert raw("tri_quantize", None, 4, 64, F2, B, C, A, need, s) == tri.TRI_EINVAL
    assert raw("tri_quantize", A, 4, 64, F2, None, C, A, need, s) == tri.TRI_EINVAL
    assert raw("tri_quantize", A, 4, 64, F2, B, None, A, need, s) == tri.TRI_EINVAL
    assert raw("tri_quantize", A, 4, 64, F2, B, C, None, need, s) == tri.TRI_EINVAL
    assert raw("tri_quantize", A, 4, 64, 2, B, C, A, need, s) == tri.TRI_EINVAL
    for (N, K) in [(0, 64), (4, 0), (1 << 31, 64), (4, 1 << 31)]:
        assert raw("tri_quantize", A, N, K, F2, B, C, A, 1 << 20, s) == tri.TRI_EINVAL
    assert raw("tri_quantize", A, 4, 64, F2, B, C, A, need - 8, s) == tri.TRI_EINVAL
    assert raw("tri_quantize", ODD, 4, 64, F2, B, C, A, need, s) == tri.TRI_EALIGN
    assert raw("tri_quantize", A, 4, 64, F2, ODD, C, A, need, s) == tri.TRI_EALIGN
    assert raw("tri_quantize", A, 4, 64, F2, B, C + 2, A, need, s) == tri.TRI_EALIGN
    assert raw("tri_quantize", A, 4, 64, F2, B, C, ODD, need, s) == tri.TRI_EALIGN
    # the allocation-free variant: the same checks without the workspace, before any device call
    assert tri.tri_quantize_workspace_bytes(28672, 8192) <= tri.TRI_QUANTIZE_SCRATCH_BYTES
    assert raw("tri_quantize_noalloc", None, 4, 64, F2, B, C, s) == tri.TRI_EINVAL
    assert raw("tri_quantize_noalloc", A, 4, 64, F2, None, C, s) == tri.TRI_EINVAL
    assert raw("tri_quantize_noalloc", A, 4, 64, F2, B, None, s) == tri.TRI_EINVAL
    assert raw("tri_quantize_noalloc", A, 4, 64, 2, B, C, s) == tri.TRI_EINVAL
    for (N, K) in [(0, 64), (4, 0), (1 << 31, 64), (4, 1 << 31)]:
        assert raw("tri_quantize_noalloc", A, N, K, F2, B, C, s) == tri.TRI_EINVAL
    assert raw("tri_quantize_noalloc", ODD, 4, 64, F2, B, C, s) == tri.TRI_EALIGN
    assert raw("tri_quantize_noalloc", A, 4, 64, F2, ODD, C, s) == tri.TRI_EALIGN
    assert raw("tri_quantize_noalloc", A, 4, 64, F2, B, C + 2, s) == tri.TRI_EALIGN


def test_fused_argument_errors_launch_nothing():
    import ctypes
    F2 = tri.TRI_FMT_2BIT
    s = None
    ptrs = lambda *v: (ctypes.c_void_p * len(v))(*v)
    floats = lambda *v: (ctypes.c_float * len(v))(*v)
    ints = lambda *v: (ctypes.c_int64 * len(v))(*v)
    wp, sc, nn, yy = ptrs(B, B), floats(1.0, 1.0), ints(4, 8), ptrs(C, C)
    glue = lambda gain=None, norm=1, eps=1e-5, pair=0, res=None: ctypes.byref(tri.TriGlue(gain, norm, eps, pair, res))
    g = glue()
    call = lambda *a: raw("tri_linear_fused", *a)
    assert call(A, wp, sc, 1, nn, 64, F2, yy, 2, None, s) == tri.TRI_EINVAL     # no glue
    assert call(A, wp, sc, 1, nn, 64, F2, yy, 0, g, s) == tri.TRI_EINVAL
    assert call(A, wp, sc, 17, nn, 64, F2, yy, 2, g, s) == tri.TRI_EINVAL       # M > 16
    assert call(A, wp, sc, 1, nn, 60, F2, yy, 2, g, s) == tri.TRI_EINVAL        # K % 8
    assert call(A, wp, sc, 1, nn, 16392, F2, yy, 2, g, s) == tri.TRI_EINVAL     # rows too long for the norm
    n44 = ints(4, 4)
    assert call(A, wp, sc, 16, n44, 8200, F2, yy, 2, glue(norm=0, pair=1), s) == tri.TRI_EINVAL   # pair, M > 8
    for eps in (-1.0, float("nan"), float("inf")):
        assert call(A, wp, sc, 1, nn, 64, F2, yy, 2, glue(eps=eps), s) == tri.TRI_EINVAL
    # pair: two matrices of the same N, no residual on the second
    assert call(A, wp, sc, 1, nn, 64, F2, yy, 2, glue(pair=1), s) == tri.TRI_EINVAL            # N differ
    assert call(A, ptrs(B, B, B), floats(1, 1, 1), 1, ints(4, 4, 4), 64, F2, ptrs(C, C, C), 3,
                glue(pair=1), s) == tri.TRI_EINVAL
    res2 = ctypes.cast(ptrs(None, C), ctypes.c_void_p).value
    assert call(A, wp, sc, 1, n44, 64, F2, yy, 2, glue(pair=1, res=res2), s) == tri.TRI_EINVAL
    # alignment
    assert call(A, wp, sc, 1, nn, 64, F2, yy, 2, glue(gain=ODD), s) == tri.TRI_EALIGN
    resodd = ctypes.cast(ptrs(None, ODD), ctypes.c_void_p).value
    assert call(A, wp, sc, 1, nn, 64, F2, yy, 2, glue(norm=0, res=resodd), s) == tri.TRI_EALIGN
    assert call(ODD, wp, sc, 1, nn, 64, F2, yy, 2, g, s) == tri.TRI_EALIGN
    assert call(A, wp, sc, 1, ints(4, 0), 64, F2, yy, 2, g, s) == tri.TRI_EINVAL
