"""GPU parity of the layer with a decode block's glue folded in (tri_linear_fused).

Every output is compared with the oracle's float64 fused layer on the same inputs,
element by element.  A single layer keeps the layer's tolerance, taken over the
effective input x' (the RMS-normalised row when the norm is on):
    |Y - Y_ref| <= e(Y) = 2e-3 * |scale| * sum_k |x'_k| + 1e-3 * |Y_ref|.
(The GPU rounds the gained activations to fp16, as an unfused RMSNorm output
would be: at most 2^-11 of each term; 1/rms is fp32.)
The pair output silu(y0) * y1 is held to the error the two layers' bounds e0, e1
can propagate through it -- silu has slope at most 1.1 -- plus its own fp16
rounding:  1.1 * e0 * (|y1| + e1) + |silu(y0)| * e1 + 1e-3 * |out_ref|.
The block step chains four fused launches and is compared with the oracle's chain
of the same fused layers.
"""
import numpy as np
import pytest

import oracle
import bit_mixed_precision_tri_amd as tri
from bit_mixed_precision_tri_amd import configs, synth
from tests.gpu_helpers import say, cuda, host

pytestmark = pytest.mark.gpu
FMTS = (tri.TRI_FMT_2BIT, tri.TRI_FMT_1P6BIT)


def effective_abs_sum(X, norm, gain, eps):
    """sum_k |x'_k| per row in float64: the scale of the tolerance (not an expected value)."""
    x = X.astype(np.float64)
    if norm:
        r = np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
        x = x * (1.0 if gain is None else gain.astype(np.float64)[None, :]) / r
    return np.abs(x).sum(axis=1, keepdims=True)


def layer_bound(X, s, norm, gain, eps, Yref):
    return 2e-3 * abs(s) * effective_abs_sum(X, norm, gain, eps) + 1e-3 * np.abs(Yref)


def assert_within(Y, Yref, tol, what):
    err = np.abs(Y.astype(np.float64) - Yref)
    bad = err > tol
    assert not bad.any(), "%s: %d of %d outside tolerance (worst %g vs %g)" % (
        what, int(bad.sum()), bad.size, float(err[bad].max()), float(tol[bad][np.argmax(err[bad])]))
    return float((err / np.maximum(tol, 1e-300)).max())


def check_layer_fused(Y, X, W, s, norm, gain, eps, R, what):
    Yref = oracle.linear_fused_f64(X, W, s, norm=norm, gain=gain, eps=eps, residual=R)
    return assert_within(Y, Yref, layer_bound(X, s, norm, gain, eps, Yref), what)


def check_pair(Y, X, Wg, sg, Wu, su, norm, gain, eps, R, what):
    y0 = oracle.linear_fused_f64(X, Wg, sg, norm=norm, gain=gain, eps=eps)
    y1 = oracle.linear_fused_f64(X, Wu, su, norm=norm, gain=gain, eps=eps)
    ref = oracle.silu_pair_f64(X, Wg, sg, Wu, su, norm=norm, gain=gain, eps=eps)
    if R is not None:
        ref = ref + R.astype(np.float64)
    e0 = layer_bound(X, sg, norm, gain, eps, y0)
    e1 = layer_bound(X, su, norm, gain, eps, y1)
    silu0 = np.abs(oracle.silu_mul_f64(y0, np.ones_like(y0)))
    tol = 1.1 * e0 * (np.abs(y1) + e1) + silu0 * e1 + 1e-3 * np.abs(ref)
    return assert_within(Y, ref, tol, what)


def run_fused(X, Wps, scales, Ns, K, fmt, norm=False, gain=None, eps=1e-5, pair=False, Rs=None, inplace=False):
    import torch
    M = X.shape[0]
    Xd = cuda(X)
    nd = None if gain is None else cuda(gain)
    if inplace:
        Ys = [cuda(R) for R in Rs]
        rd = Ys
    else:
        Ys = [torch.empty((M, N), dtype=torch.float16, device="cuda") for N in Ns]
        rd = None if Rs is None else [None if R is None else cuda(R) for R in Rs]
    if pair:
        Ys[1] = None
    tri.tri_linear_fused(Xd, Wps, scales, M, Ns, K, fmt, Ys, norm=norm, gain=nd, eps=eps, pair=pair, residuals=rd)
    return [None if Y is None else host(Y) for Y in Ys]


SINGLE = [
    dict(name="norm", norm=True),
    dict(name="norm+gain", norm=True, gain=True),
    dict(name="residual", res=True),
    dict(name="norm+gain+residual", norm=True, gain=True, res=True),
]
PAIRED = [
    dict(name="pair", pair=True),
    dict(name="pair+norm+gain", pair=True, norm=True, gain=True),
    dict(name="pair+norm+residual", pair=True, norm=True, res=True),
]
SHAPES = [(1, 4096), (2, 4096), (3, 1000), (8, 11008), (16, 4096), (1, 11008), (12, 1000)]


def inputs(M, K, Ns, seed):
    rng = synth.rng_for(seed, M, K)
    Ws = [synth.trits(rng, N, K) for N in Ns]
    scales = [synth.uniform_scale(rng) for _ in Ns]
    X = synth.activations(rng, M, K)
    gain = (1 + 0.1 * synth.activations(rng, 1, K)[0]).astype(np.float16)
    Rs = [synth.activations(rng, M, N) for N in Ns]
    return Ws, scales, X, gain, Rs


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", SHAPES, ids=["M%d_K%d" % s for s in SHAPES])
def test_fused_single_layers(fmt, shape):
    M, K = shape
    Ns = [37, 256, 100]
    Ws, scales, X, gain, Rs = inputs(M, K, Ns, 980)
    Wps = [tri.pack(cuda(W), fmt) for W in Ws]
    worst = 0.0
    for opt in SINGLE:
        norm = bool(opt.get("norm"))
        gn = gain if opt.get("gain") else None
        R = Rs if opt.get("res") else None
        Ys = run_fused(X, Wps, scales, Ns, K, fmt, norm=norm, gain=gn, Rs=R)
        for g in range(len(Ns)):
            what = "M=%d K=%d fmt=%d %s matrix %d" % (M, K, fmt, opt["name"], g)
            worst = max(worst, check_layer_fused(Ys[g], X, Ws[g], scales[g], norm, gn, 1e-5,
                                                 None if R is None else R[g], what))
    say("M=%d K=%d fmt=%d: worst error / tolerance %.3f" % (M, K, fmt, worst))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", SHAPES, ids=["M%d_K%d" % s for s in SHAPES])
def test_fused_silu_pair(fmt, shape):
    M, K = shape
    if M > 8 and K > (8192 if fmt == tri.TRI_FMT_2BIT else 10240):
        pytest.skip("pair with more than 8 rows serves shorter rows")
    Ns = [300, 300]
    Ws, scales, X, gain, Rs = inputs(M, K, Ns, 983)
    Wps = [tri.pack(cuda(W), fmt) for W in Ws]
    worst = 0.0
    for opt in PAIRED:
        norm = bool(opt.get("norm"))
        gn = gain if opt.get("gain") else None
        R = [Rs[0], None] if opt.get("res") else None
        Y = run_fused(X, Wps, scales, Ns, K, fmt, norm=norm, gain=gn, pair=True, Rs=R)[0]
        what = "M=%d K=%d fmt=%d %s" % (M, K, fmt, opt["name"])
        worst = max(worst, check_pair(Y, X, Ws[0], scales[0], Ws[1], scales[1], norm, gn, 1e-5,
                                      None if R is None else R[0], what))
    say("pair M=%d K=%d fmt=%d: worst error / tolerance %.3f" % (M, K, fmt, worst))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,K", [(5, 1000), (8, 4096), (6, 4000)])
def test_fused_silu_pair_two_block_workgroups(fmt, M, K):
    """Gate and up of 5150 rows: at least 160 workgroups of two 16-row blocks of each matrix, so the
    batched kernel's pair variant takes two blocks per workgroup; the last workgroup holds a full
    block and one of 14 rows."""
    Ns = [5150, 5150]
    Ws, scales, X, gain, Rs = inputs(M, K, Ns, 986)
    Wps = [tri.pack(cuda(W), fmt) for W in Ws]
    worst = 0.0
    for opt in PAIRED:
        norm = bool(opt.get("norm"))
        gn = gain if opt.get("gain") else None
        R = [Rs[0], None] if opt.get("res") else None
        say("pair two blocks M=%d K=%d fmt=%d %s" % (M, K, fmt, opt["name"]))
        Y = run_fused(X, Wps, scales, Ns, K, fmt, norm=norm, gain=gn, pair=True, Rs=R)[0]
        what = "two-block pair M=%d K=%d fmt=%d %s" % (M, K, fmt, opt["name"])
        worst = max(worst, check_pair(Y, X, Ws[0], scales[0], Ws[1], scales[1], norm, gn, 1e-5,
                                      None if R is None else R[0], what))
    say("pair two blocks M=%d K=%d fmt=%d: worst error / tolerance %.3f" % (M, K, fmt, worst))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [4, 8, 16])
def test_fused_norm_multi_block_workgroups(fmt, M):
    """Grids large enough for workgroups of several 16-row blocks (4096 + 4096 + 2000 rows): the
    norm variant with the gain and a residual, ragged last block."""
    K = 1000
    Ns = [4096, 4096, 2000]
    Ws, scales, X, gain, Rs = inputs(M, K, Ns, 985)
    Wps = [tri.pack(cuda(W), fmt) for W in Ws]
    Ys = run_fused(X, Wps, scales, Ns, K, fmt, norm=True, gain=gain, Rs=Rs)
    worst = 0.0
    for g in range(len(Ns)):
        worst = max(worst, check_layer_fused(Ys[g], X, Ws[g], scales[g], True, gain, 1e-5, Rs[g],
                                             "multi-block M=%d fmt=%d matrix %d" % (M, fmt, g)))
    say("multi-block norm M=%d fmt=%d: worst error / tolerance %.3f" % (M, fmt, worst))


@pytest.mark.parametrize("fmt", FMTS)
def test_fused_without_glue_equals_grouped_bitwise(fmt):
    import torch
    for (M, K) in [(1, 4096), (2, 4096), (5, 1000), (16, 11008)]:
        Ns = [64, 300]
        Ws, scales, X, _, _ = inputs(M, K, Ns, 981)
        Wps = [tri.pack(cuda(W), fmt) for W in Ws]
        Yf = run_fused(X, Wps, scales, Ns, K, fmt)
        Xd = cuda(X)
        Yg = [torch.empty((M, N), dtype=torch.float16, device="cuda") for N in Ns]
        tri.tri_linear_grouped(Xd, Wps, scales, M, Ns, K, fmt, Yg)
        for a, b in zip(Yf, Yg):
            np.testing.assert_array_equal(a.view(np.uint16), host(b).view(np.uint16))


@pytest.mark.parametrize("fmt", FMTS)
def test_fused_in_place_residual_and_zero_rows(fmt):
    M, K, N = 4, 4096, 200
    Ws, scales, X, _, Rs = inputs(M, K, [N], 982)
    X[2] = 0                                     # a zero row under the norm: 1/sqrt(eps) * 0
    Wp = tri.pack(cuda(Ws[0]), fmt)
    Y = run_fused(X, [Wp], scales, [N], K, fmt, norm=True, eps=1e-5, Rs=Rs, inplace=True)[0]
    check_layer_fused(Y, X, Ws[0], scales[0], True, None, 1e-5, Rs[0], "in-place residual fmt=%d" % fmt)
    np.testing.assert_array_equal(Y[2], Rs[0][2])   # the zero row leaves exactly the residual


def block_chain(x, layers, fmt, gpu):
    """One decode block as four fused layers (each of the M rows a sequence at its first position,
    so attention returns V):  q,k,v = QKV(rmsnorm(x));  h = x + O(v);  a = silu(gate(rmsnorm(h))) *
    up(rmsnorm(h));  out = h + down(a).  gpu=False evaluates every layer with the oracle (float64,
    rounded to fp16 like the GPU's outputs).  Returns the output and each launch's input."""
    eps = 1e-5
    inputs_ = {}

    def fused(names, X, norm=False, pair=False, R=None):
        Ws = [layers[n] for n in names]
        inputs_[names[0]] = (X, R)
        if gpu:
            return run_fused(X, [w[1] for w in Ws], [w[2] for w in Ws], [w[0].shape[0] for w in Ws], X.shape[1], fmt,
                             norm=norm, eps=eps, pair=pair, Rs=None if R is None else [R] + [None] * (len(Ws) - 1))
        if pair:
            return [oracle.silu_pair_f64(X, Ws[0][0], Ws[0][2], Ws[1][0], Ws[1][2], norm=norm,
                                         eps=eps).astype(np.float16), None]
        return [oracle.linear_fused_f64(X, w[0], w[2], norm=norm, eps=eps, residual=R).astype(np.float16)
                for w in Ws]

    q, k, v = fused(["q", "k", "v"], x, norm=True)
    h, = fused(["o"], v, R=x)
    a, _ = fused(["gate", "up"], h, norm=True, pair=True)
    out, = fused(["down"], a, R=h)
    return out, inputs_


@pytest.mark.parametrize("M", [1, 8])
def test_block_step_fused(M):
    """The decode block as four fused launches (QKV with the norm, O + residual, gate/up with the
    norm and the silu gate, down + residual): every launch is checked on the oracle chain's
    inputs, and the whole chain against the oracle's chain."""
    cfg = configs.BLOCK
    fmt = cfg["fmt"]
    layers = {}
    for li, (name, K, N) in enumerate(cfg["layers"]):
        W = synth.trits(synth.rng_for(cfg["workload_id"], li, synth.STREAM_W), N, K)
        s = synth.uniform_scale(synth.rng_for(cfg["workload_id"], li, synth.STREAM_SCALE))
        layers[name] = (W, tri.pack(cuda(W), fmt), s)
    x0 = synth.activations(synth.rng_for(cfg["workload_id"], 100 + M, synth.STREAM_X), M, cfg["hidden"])
    out_ref, ins = block_chain(x0, layers, fmt, gpu=False)
    out_gpu, _ = block_chain(x0, layers, fmt, gpu=True)
    eps = 1e-5
    for first, names, norm in (("q", ["q", "k", "v"], True), ("o", ["o"], False), ("down", ["down"], False)):
        X, R = ins[first]
        Ys = run_fused(X, [layers[n][1] for n in names], [layers[n][2] for n in names],
                       [layers[n][0].shape[0] for n in names], X.shape[1], fmt, norm=norm, eps=eps,
                       Rs=None if R is None else [R])
        for n, Y in zip(names, Ys):
            check_layer_fused(Y, X, layers[n][0], layers[n][2], norm, None, eps, R, "block M=%d %s" % (M, n))
    X, _ = ins["gate"]
    Wg, Wu = layers["gate"], layers["up"]
    Y = run_fused(X, [Wg[1], Wu[1]], [Wg[2], Wu[2]], [Wg[0].shape[0]] * 2, X.shape[1], fmt, norm=True, eps=eps,
                  pair=True)[0]
    check_pair(Y, X, Wg[0], Wg[2], Wu[0], Wu[2], True, None, eps, None, "block M=%d gate/up" % M)
    a, b = out_gpu.astype(np.float64), out_ref.astype(np.float64)
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    say("fused block M=%d: relative difference of the GPU chain to the oracle chain %.3g" % (M, rel))
    assert rel < 1e-2


@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("fmt", FMTS)
def test_fused_residual_tall_matrix(fmt, M):
    """One tall matrix with a residual: the decode kernel's block loop adds the residual when it
    writes its outputs out (separate and in-place residual)."""
    N, K = 40007, 4096
    W, X, s = synth.layer_inputs(530 + fmt, 1, M, N, K)
    R = synth.activations(synth.rng_for(530 + fmt, 2, synth.STREAM_X), M, N)
    Wp = tri.pack(cuda(W), fmt)
    say("fused residual tall M=%d N=%d fmt=%d" % (M, N, fmt))
    for inplace in (False, True):
        Y = run_fused(X, [Wp], [s], [N], K, fmt, Rs=[R], inplace=inplace)[0]
        check_layer_fused(Y, X, W, s, False, None, 1e-5, R, "tall residual fmt=%d inplace=%s" % (fmt, inplace))
