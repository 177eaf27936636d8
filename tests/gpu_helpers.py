"""Shared helpers of the GPU parity tests (test infrastructure, not product code)."""
import sys

import numpy as np

import oracle
import bit_mixed_precision_tri_amd as tri


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def cuda(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def algos_for(M, fmt):
    """Kernel families that can serve (M, fmt)."""
    out = [tri.TRI_ALGO_GEMM, tri.TRI_ALGO_SMALLM]
    if M == 1 and fmt == tri.TRI_FMT_2BIT:
        out.append(tri.TRI_ALGO_GEMV)
    return out


def check_layer(Y_gpu, X, W, scale, what="", rows=None):
    """Element-wise check of fp16 Y_gpu against the oracle:
    |Y - Y_ref| <= 2e-3*|scale|*sum_k|x_k| + 1e-3*|Y_ref| for every element.
    `rows` restricts the check to those rows of X (Y_gpu holds all rows).
    Returns (max err/tol, fraction equal to fp16(Y_ref))."""
    Xs = X if rows is None else X[rows]
    Yg = (Y_gpu if rows is None else Y_gpu[rows]).astype(np.float64)
    Yref = oracle.linear_f64(Xs, W, scale)
    tol = oracle.tolerance(Xs, scale, Yref)
    err = np.abs(Yg - Yref)
    ratio = err / tol
    worst = float(ratio.max())
    if not np.all(err <= tol):
        i = np.unravel_index(np.argmax(ratio), ratio.shape)
        raise AssertionError("%s: %d elements out of tolerance; worst at %s: gpu %r ref %r tol %r"
                             % (what, int((err > tol).sum()), i, Yg[i], Yref[i], tol[i]))
    exact = float(np.mean(Yg == Yref.astype(np.float16).astype(np.float64)))
    return worst, exact
