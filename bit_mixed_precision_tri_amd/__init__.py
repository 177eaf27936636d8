"""Python binding of libtri, the gfx950 ternary linear layer.

The functions named ``tri_*`` mirror the C ABI in ``include/tri.h`` one to one:
they only marshal arguments (device pointers of torch tensors, the current HIP
stream) and raise ``TriError`` on a negative status.  All the work runs in the
library's HIP kernels; there is no fallback of any kind -- if ``libtri.so`` is
missing, every call raises.  The helpers at the end (``pack``, ``unpack``,
``quantize``, ``linear``) allocate their outputs with torch and then call the same
entry points.
"""
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libtri.so")

TRI_FMT_2BIT = 0
TRI_FMT_1P6BIT = 1
TRI_OK, TRI_EINVAL, TRI_EALIGN, TRI_EHIP = 0, -1, -2, -3
TRI_ALGO_AUTO, TRI_ALGO_GEMV, TRI_ALGO_SMALLM, TRI_ALGO_GEMM = 0, 1, 2, 3
ALGO_NAMES = {TRI_ALGO_GEMV: "gemv", TRI_ALGO_SMALLM: "smallm", TRI_ALGO_GEMM: "gemm"}

_lib = None


class TriGlue(ctypes.Structure):
    """tri_glue of include/tri.h."""
    _fields_ = [("norm_gain", ctypes.c_void_p), ("norm", ctypes.c_int), ("norm_eps", ctypes.c_float),
                ("pair", ctypes.c_int), ("residual", ctypes.c_void_p)]


class TriError(RuntimeError):
    def __init__(self, code, what):
        super().__init__("%s failed: %s (%d)" % (what, status_string(code), code))
        self.code = code


def lib():
    """The loaded libtri.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libtri.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        i64, p, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.tri_row_bytes.argtypes = [i64, i32]
        L.tri_row_bytes.restype = i64
        for name in ("tri_pack2", "tri_pack16"):
            getattr(L, name).argtypes = [p, i64, i64, p, p]
            getattr(L, name).restype = i32
        L.tri_unpack.argtypes = [p, i64, i64, i32, p, p]
        L.tri_unpack.restype = i32
        L.tri_quantize_workspace_bytes.argtypes = [i64, i64]
        L.tri_quantize_workspace_bytes.restype = i64
        L.tri_quantize.argtypes = [p, i64, i64, i32, p, p, p, i64, p]
        L.tri_quantize.restype = i32
        L.tri_quantize_noalloc.argtypes = [p, i64, i64, i32, p, p, p]
        L.tri_quantize_noalloc.restype = i32
        L.tri_linear.argtypes = [p, p, ctypes.c_float, i64, i64, i64, i32, p, p]
        L.tri_linear.restype = i32
        L.tri_linear_algo.argtypes = [p, p, ctypes.c_float, i64, i64, i64, i32, p, i32, p]
        L.tri_linear_algo.restype = i32
        L.tri_linear_grouped.argtypes = [p, p, p, i64, p, i64, i32, p, i32, p]
        L.tri_linear_grouped.restype = i32
        L.tri_linear_fused.argtypes = [p, p, p, i64, p, i64, i32, p, i32, ctypes.POINTER(TriGlue), p]
        L.tri_linear_fused.restype = i32
        L.tri_select_algo.argtypes = [i64, i64, i64, i32]
        L.tri_select_algo.restype = i32
        L.tri_status_string.argtypes = [i32]
        L.tri_status_string.restype = ctypes.c_char_p
        L.tri_probe_read.argtypes = [p, i64, p, p]
        L.tri_probe_read.restype = i32
        L.tri_probe_copy.argtypes = [p, p, i64, p]
        L.tri_probe_copy.restype = i32
        L.tri_probe_empty.argtypes = [i64, i32, p, p]
        L.tri_probe_empty.restype = i32
        L.tri_probe_rows.argtypes = [p, p, i64, i64, i32, i32, p, p]
        L.tri_probe_rows.restype = i32
        L.tri_probe_stream.argtypes = [p, i64, i32, i32, p, p]
        L.tri_probe_stream.restype = i32
        _lib = L
    return _lib


def status_string(code):
    return lib().tri_status_string(int(code)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr() if hasattr(t, "data_ptr") else int(t))


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(rc, what):
    if rc != TRI_OK:
        raise TriError(rc, what)
    return rc


# ---------------------------------------------------------------- the C ABI, one to one

def tri_row_bytes(K, fmt):
    return int(lib().tri_row_bytes(int(K), int(fmt)))


def tri_pack2(W, N, K, Wp, stream=None):
    return _check(lib().tri_pack2(_ptr(W), int(N), int(K), _ptr(Wp), _stream(stream)), "tri_pack2")


def tri_pack16(W, N, K, Wp, stream=None):
    return _check(lib().tri_pack16(_ptr(W), int(N), int(K), _ptr(Wp), _stream(stream)), "tri_pack16")


def tri_unpack(Wp, N, K, fmt, W, stream=None):
    return _check(lib().tri_unpack(_ptr(Wp), int(N), int(K), int(fmt), _ptr(W), _stream(stream)), "tri_unpack")


def tri_quantize_workspace_bytes(N, K):
    return int(lib().tri_quantize_workspace_bytes(int(N), int(K)))


def tri_quantize(W, N, K, fmt, Wp, scale_out, workspace, workspace_bytes, stream=None):
    return _check(lib().tri_quantize(_ptr(W), int(N), int(K), int(fmt), _ptr(Wp), _ptr(scale_out), _ptr(workspace),
                                     int(workspace_bytes), _stream(stream)), "tri_quantize")


def tri_quantize_noalloc(W, N, K, fmt, Wp, scale_out, stream=None):
    return _check(lib().tri_quantize_noalloc(_ptr(W), int(N), int(K), int(fmt), _ptr(Wp), _ptr(scale_out),
                                             _stream(stream)), "tri_quantize_noalloc")


def tri_linear(X, Wp, scale, M, N, K, fmt, Y, stream=None):
    return _check(lib().tri_linear(_ptr(X), _ptr(Wp), float(scale), int(M), int(N), int(K), int(fmt), _ptr(Y),
                                   _stream(stream)), "tri_linear")


def tri_linear_algo(X, Wp, scale, M, N, K, fmt, Y, algo, stream=None):
    return _check(lib().tri_linear_algo(_ptr(X), _ptr(Wp), float(scale), int(M), int(N), int(K), int(fmt), _ptr(Y),
                                        int(algo), _stream(stream)), "tri_linear_algo")


TRI_MAX_GROUPS = 4
TRI_QUANTIZE_SCRATCH_BYTES = 16384


def tri_linear_grouped(X, Wps, scales, M, Ns, K, fmt, Ys, stream=None):
    """Wps, scales, Ns, Ys: sequences of G entries (device tensors / floats / ints)."""
    G = len(Wps)
    if not (len(scales) == len(Ns) == len(Ys) == G):
        raise ValueError("tri_linear_grouped: Wps, scales, Ns and Ys must have the same length")
    wp = (ctypes.c_void_p * max(G, 1))(*[_ptr(w).value for w in Wps])
    sc = (ctypes.c_float * max(G, 1))(*[float(v) for v in scales])
    nn = (ctypes.c_int64 * max(G, 1))(*[int(v) for v in Ns])
    yy = (ctypes.c_void_p * max(G, 1))(*[_ptr(y).value for y in Ys])
    return _check(lib().tri_linear_grouped(_ptr(X), wp, sc, int(M), nn, int(K), int(fmt), yy, int(G),
                                           _stream(stream)), "tri_linear_grouped")


def tri_linear_fused(X, Wps, scales, M, Ns, K, fmt, Ys, norm=False, gain=None, eps=1e-5, pair=False,
                     residuals=None, stream=None):
    """tri_linear_grouped with a decode block's glue: y_g = scales[g] * x' W_g^T (x' = rmsnorm(X) if norm);
    Ys[g] = fp16(residuals[g] + y_g), or with pair (two matrices, gate then up) Ys[0] = fp16(residuals[0] +
    silu(y_0) * y_1).  residuals: None or a sequence of G entries (tensor or None); Ys[1] may be None with pair."""
    G = len(Wps)
    if not (len(scales) == len(Ns) == len(Ys) == G) or (residuals is not None and len(residuals) != G):
        raise ValueError("tri_linear_fused: per-matrix sequences must have the same length")
    wp = (ctypes.c_void_p * max(G, 1))(*[_ptr(w).value for w in Wps])
    sc = (ctypes.c_float * max(G, 1))(*[float(v) for v in scales])
    nn = (ctypes.c_int64 * max(G, 1))(*[int(v) for v in Ns])
    yy = (ctypes.c_void_p * max(G, 1))(*[None if y is None else _ptr(y).value for y in Ys])
    rr = None
    if residuals is not None:
        rr = (ctypes.c_void_p * max(G, 1))(*[None if r is None else _ptr(r).value for r in residuals])
    glue = TriGlue(None if gain is None else _ptr(gain).value, 1 if norm else 0, float(eps), 1 if pair else 0,
                   None if rr is None else ctypes.cast(rr, ctypes.c_void_p).value)
    return _check(lib().tri_linear_fused(_ptr(X), wp, sc, int(M), nn, int(K), int(fmt), yy, int(G),
                                         ctypes.byref(glue), _stream(stream)), "tri_linear_fused")


def tri_select_algo(M, N, K, fmt):
    return int(lib().tri_select_algo(int(M), int(N), int(K), int(fmt)))


def tri_status_string(code):
    return status_string(code)


def tri_probe_read(src, nbytes, sink, stream=None):
    return _check(lib().tri_probe_read(_ptr(src), int(nbytes), _ptr(sink), _stream(stream)), "tri_probe_read")


def tri_probe_copy(src, dst, nbytes, stream=None):
    return _check(lib().tri_probe_copy(_ptr(src), _ptr(dst), int(nbytes), _stream(stream)), "tri_probe_copy")


def tri_probe_empty(workgroups, threads, sink, stream=None):
    return _check(lib().tri_probe_empty(int(workgroups), int(threads), _ptr(sink), _stream(stream)), "tri_probe_empty")


def tri_probe_rows(X, Wp, N, K, fmt, waves, Y, stream=None):
    return _check(lib().tri_probe_rows(_ptr(X), _ptr(Wp), int(N), int(K), int(fmt), int(waves), _ptr(Y),
                                       _stream(stream)), "tri_probe_rows")


def tri_probe_stream(src, nbytes, workgroups, unroll, sink, stream=None):
    return _check(lib().tri_probe_stream(_ptr(src), int(nbytes), int(workgroups), int(unroll), _ptr(sink),
                                         _stream(stream)), "tri_probe_stream")


# ---------------------------------------------------------------- allocating helpers

def pack(W, fmt, stream=None):
    """Pack a (N, K) int8 CUDA tensor; returns a new (N, row_bytes) uint8 tensor."""
    import torch
    N, K = W.shape
    assert W.dtype == torch.int8 and W.is_cuda and W.is_contiguous()
    Wp = torch.empty((N, tri_row_bytes(K, fmt)), dtype=torch.uint8, device=W.device)
    (tri_pack2 if fmt == TRI_FMT_2BIT else tri_pack16)(W, N, K, Wp, stream)
    return Wp


def unpack(Wp, K, fmt, stream=None):
    """Unpack a (N, row_bytes) uint8 CUDA tensor; returns a new (N, K) int8 tensor."""
    import torch
    N = Wp.shape[0]
    assert Wp.dtype == torch.uint8 and Wp.is_cuda and Wp.is_contiguous()
    assert Wp.shape[1] == tri_row_bytes(K, fmt)
    W = torch.empty((N, K), dtype=torch.int8, device=Wp.device)
    tri_unpack(Wp, N, K, fmt, W, stream)
    return W


def quantize(W, fmt, stream=None):
    """Quantise a (N, K) float32 CUDA tensor of latent weights; returns (packed weights as a new
    (N, row_bytes) uint8 tensor, the scale as a new 1-element float32 tensor on the device)."""
    import torch
    N, K = W.shape
    assert W.dtype == torch.float32 and W.is_cuda and W.is_contiguous()
    Wp = torch.empty((N, tri_row_bytes(K, fmt)), dtype=torch.uint8, device=W.device)
    scale = torch.empty(1, dtype=torch.float32, device=W.device)
    nbytes = tri_quantize_workspace_bytes(N, K)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=W.device)
    tri_quantize(W, N, K, fmt, Wp, scale, ws, nbytes, stream)
    return Wp, scale


def linear(X, Wp, scale, K, fmt, algo=TRI_ALGO_AUTO, out=None, stream=None):
    """Y = fp16(scale * X @ W.T) for a (M, K) fp16 CUDA tensor X and packed weights Wp."""
    import torch
    M = X.shape[0]
    N = Wp.shape[0]
    assert X.dtype == torch.float16 and X.is_cuda and X.is_contiguous() and X.shape[1] == K
    assert Wp.dtype == torch.uint8 and Wp.is_contiguous() and Wp.shape[1] == tri_row_bytes(K, fmt)
    Y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=X.device)
    if algo == TRI_ALGO_AUTO:
        tri_linear(X, Wp, scale, M, N, K, fmt, Y, stream)
    else:
        tri_linear_algo(X, Wp, scale, M, N, K, fmt, Y, algo, stream)
    return Y
