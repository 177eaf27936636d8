"""CPU oracle for the ternary linear layer -- TEST INFRASTRUCTURE ONLY.

This package wraps ``tri_oracle.c``: a plain, slow, scalar C implementation of
the 2-bit and 1.6-bit packings, their inverse, the ternary linear layer
``Y = scale * (X @ W.T)`` summed in float64 (also with a decode block's glue --
RMSNorm, residual, SiLU gate of two layers -- folded around it), and the quantiser
from latent float32 weights to trits and a scale.  It exists to check the HIP library,
and only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import it.  It shares no code with the HIP library (the only
common module is the seeded input generator, which holds none of the layer's
arithmetic).

Sources: the web pages on Spectra 1.1 (arXiv 2506.23025) -- the pith.science
review ("What carries the argument", "Core claim", "Referee Report" minor
comment 5, "Significance") and the shd-paper.top summary (abstract).  The C
source states every reading taken where the pages are silent.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tri_oracle.c")
_LIB_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_LIB_DIR, "liboracle.so")

FMT_2BIT = 0
FMT_1P6BIT = 1

_lib = None


def build(force=False):
    """Compile tri_oracle.c with gcc (-O2, no fast-math, OpenMP) into oracle/_build."""
    os.makedirs(_LIB_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-shared", "-fPIC",
                               "-Wall", "-Werror", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        override = os.environ.get("TRI_ORACLE_LIB")   # a planted-mistake build, used by the mutation test
        if override:
            lib = ctypes.CDLL(override)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            lib = ctypes.CDLL(_LIB)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_row_bytes.argtypes = [i64, ctypes.c_int]
        lib.oracle_row_bytes.restype = i64
        lib.oracle_pack2.argtypes = [p, i64, i64, p]
        lib.oracle_pack2.restype = None
        lib.oracle_pack16.argtypes = [p, i64, i64, p]
        lib.oracle_pack16.restype = None
        lib.oracle_unpack.argtypes = [p, i64, i64, ctypes.c_int, p]
        lib.oracle_unpack.restype = ctypes.c_int
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_half_to_double.restype = ctypes.c_double
        lib.oracle_linear_f64.argtypes = [p, p, ctypes.c_double, i64, i64, i64, p, ctypes.c_int]
        lib.oracle_linear_f64.restype = ctypes.c_int
        lib.oracle_quantize.argtypes = [p, i64, i64, p, p]
        lib.oracle_quantize.restype = ctypes.c_int
        lib.oracle_linear_fused_f64.argtypes = [p, ctypes.c_int, p, ctypes.c_double, p, ctypes.c_double, p,
                                                i64, i64, i64, p]
        lib.oracle_silu_mul_f64.argtypes = [p, p, i64, p]
        lib.oracle_silu_mul_f64.restype = None
        lib.oracle_linear_fused_f64.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def row_bytes(K, fmt):
    """Bytes of one packed row (16*ceil(K/64) for 2-bit, 16*ceil(K/80) for 1.6-bit)."""
    return int(_load().oracle_row_bytes(int(K), int(fmt)))


def pack(W, fmt):
    """Pack an (N, K) int8 matrix of trits (any int8; sign is encoded) -> (N, row_bytes) uint8."""
    W = np.ascontiguousarray(W, dtype=np.int8)
    N, K = W.shape
    S = row_bytes(K, fmt)
    if S < 0:
        raise ValueError("bad K or fmt")
    out = np.empty((N, S), dtype=np.uint8)
    if N:
        (_load().oracle_pack2 if fmt == FMT_2BIT else _load().oracle_pack16)(_ptr(W), N, K, _ptr(out))
    return out


def pack2(W):
    return pack(W, FMT_2BIT)


def pack16(W):
    return pack(W, FMT_1P6BIT)


def unpack(Wp, K, fmt):
    """Unpack an (N, row_bytes) uint8 matrix -> (N, K) int8 trits."""
    Wp = np.ascontiguousarray(Wp, dtype=np.uint8)
    N = Wp.shape[0]
    if Wp.shape[1] != row_bytes(K, fmt):
        raise ValueError("packed row length does not match K")
    out = np.empty((N, K), dtype=np.int8)
    if N and _load().oracle_unpack(_ptr(Wp), N, K, int(fmt), _ptr(out)) != 0:
        raise ValueError("unknown format")
    return out


def half_to_double(bits):
    """Decode one fp16 bit pattern (int) to a Python float, by the oracle's own decoder."""
    return float(_load().oracle_half_to_double(int(bits) & 0xFFFF))


def linear_f64(X, W, scale, nthreads=0):
    """Y_ref = scale * (X @ W.T), summed in float64 in k order, unrounded.

    X: (M, K) float16; W: (N, K) int8 trits; scale: float (the fp32 scale).
    Returns (M, N) float64."""
    X = np.ascontiguousarray(X, dtype=np.float16)
    W = np.ascontiguousarray(W, dtype=np.int8)
    M, K = X.shape
    N, K2 = W.shape
    if K != K2:
        raise ValueError("K mismatch")
    Y = np.empty((M, N), dtype=np.float64)
    if M and N:
        rc = _load().oracle_linear_f64(_ptr(X.view(np.uint16)), _ptr(W), float(scale),
                                       M, N, K, _ptr(Y), int(nthreads))
        if rc != 0:
            raise ValueError("non-finite activation")
    return Y


def linear_packed_f64(X, Wp, K, fmt, scale, nthreads=0):
    """The layer evaluated from the packed weights: unpack, then linear_f64."""
    return linear_f64(X, unpack(Wp, K, fmt), scale, nthreads)


def quantize(W):
    """Latent float32 weights (N, K) -> (trits (N, K) int8, float32 scale): the scale is the
    float64 mean of |w| rounded to float32, a trit is round-half-even(w / scale) clipped to [-1, 1]."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    T = np.empty((N, K), dtype=np.int8)
    s = np.zeros(1, dtype=np.float32)
    if N and K and _load().oracle_quantize(_ptr(W), N, K, _ptr(T), _ptr(s)) != 0:
        raise ValueError("non-finite weight")
    return T, np.float32(s[0])


def linear_fused_f64(X, W, scale, norm=False, gain=None, eps=1e-5, residual=None):
    """The layer with block glue folded around it, in float64, unrounded:
    x2 = X * gain / sqrt(mean(X^2) + eps) per row (if norm; gain None = 1),
    Y = residual + scale * x2 @ W.T (residual None = 0).  X: (M, K) fp16; gain: (K,) fp16;
    residual: (M, N) fp16; W: (N, K) int8.  Returns (M, N) float64."""
    X = np.ascontiguousarray(X, dtype=np.float16)
    W = np.ascontiguousarray(W, dtype=np.int8)
    M, K = X.shape
    N, K2 = W.shape
    if K != K2:
        raise ValueError("K mismatch")
    gn = None if gain is None else np.ascontiguousarray(gain, dtype=np.float16).reshape(-1)
    if gn is not None and gn.shape != (K,):
        raise ValueError("gain shape")
    r = None if residual is None else np.ascontiguousarray(residual, dtype=np.float16)
    if r is not None and r.shape != (M, N):
        raise ValueError("residual shape")
    Y = np.empty((M, N), dtype=np.float64)
    opt = lambda a: None if a is None else _ptr(a.view(np.uint16))
    if M and N:
        rc = _load().oracle_linear_fused_f64(_ptr(X.view(np.uint16)), int(bool(norm)), opt(gn), float(eps),
                                             _ptr(W), float(scale), opt(r), M, N, K, _ptr(Y))
        if rc != 0:
            raise ValueError("non-finite input")
    return Y


def silu_mul_f64(a, b):
    """silu(a) * b elementwise in float64, silu(z) = z / (1 + exp(-z))."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    b = np.ascontiguousarray(b, dtype=np.float64)
    if a.shape != b.shape:
        raise ValueError("shape mismatch")
    out = np.empty_like(a)
    if a.size:
        _load().oracle_silu_mul_f64(_ptr(a), _ptr(b), a.size, _ptr(out))
    return out


def silu_pair_f64(X, W_gate, scale_gate, W_up, scale_up, norm=False, gain=None, eps=1e-5):
    """The gated-MLP input of a block: silu(gate layer) * (up layer), both layers on the same
    (optionally RMS-normalised) activations, in float64, unrounded.  Returns (M, N) float64."""
    a = linear_fused_f64(X, W_gate, scale_gate, norm=norm, gain=gain, eps=eps)
    b = linear_fused_f64(X, W_up, scale_up, norm=norm, gain=gain, eps=eps)
    return silu_mul_f64(a, b)


def max_threads():
    return int(_load().oracle_max_threads())


def tolerance(X, scale, Y_ref):
    """Per-element bound |Y - Y_ref| <= 2e-3*|scale|*sum_k|x_k| + 1e-3*|Y_ref|  (shape (M, N))."""
    sx = np.abs(np.asarray(X, dtype=np.float64)).sum(axis=1, keepdims=True)
    return 2e-3 * abs(float(scale)) * sx + 1e-3 * np.abs(Y_ref)
