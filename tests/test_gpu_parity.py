"""GPU parity: libtri (HIP, gfx950) against the CPU oracle, element by element.

Packing and unpacking must be bit-exact; the layer must satisfy, for every
element, |Y - Y_ref| <= 2e-3*|scale|*sum_k|x_k| + 1e-3*|Y_ref| with Y_ref the
unrounded float64 oracle value.  Every input is seeded (PCG64, [workload, layer,
stream]); the shapes are those of the synthetic workloads plus ragged ones.
"""
import numpy as np
import pytest

import oracle
import bit_mixed_precision_tri_amd as tri
from bit_mixed_precision_tri_amd import configs, synth
from tests.gpu_helpers import say, cuda, host, algos_for, check_layer
from tests import block_glue

pytestmark = pytest.mark.gpu

F2, F16 = tri.TRI_FMT_2BIT, tri.TRI_FMT_1P6BIT
FMTS = [F2, F16]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tri.lib()
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------- packing

@pytest.mark.parametrize("fmt", FMTS)
def test_pack_bit_exact_ragged(fmt):
    rng = synth.rng_for(100, fmt, 0)
    for N in (1, 3, 37):
        for K in (1, 2, 3, 4, 5, 6, 63, 64, 65, 79, 80, 81, 159, 160, 161, 512, 1000, 4095, 4097, 11008):
            W = synth.trits(rng, N, K)
            W[0, :: 7] = rng.integers(-128, 128, W[0, :: 7].shape)     # any int8: the sign is encoded
            got = host(tri.pack(cuda(W), fmt))
            np.testing.assert_array_equal(got, oracle.pack(W, fmt), err_msg="N=%d K=%d" % (N, K))


@pytest.mark.parametrize("fmt", FMTS)
def test_unpack_every_byte_value_bit_exact(fmt):
    K = 4 if fmt == F2 else 5
    S = tri.tri_row_bytes(K, fmt)
    Wp = np.zeros((256, S), np.uint8)
    Wp[:, 0] = np.arange(256)
    Wp[:, 1:] = np.arange(256)[::-1, None]       # every byte value in the padding too
    got = host(tri.unpack(cuda(Wp), K, fmt))
    np.testing.assert_array_equal(got, oracle.unpack(Wp, K, fmt))
    Kfull = S * (4 if fmt == F2 else 5)          # decode the whole row, all 256 values per position
    np.testing.assert_array_equal(host(tri.unpack(cuda(Wp), Kfull, fmt)), oracle.unpack(Wp, Kfull, fmt))


@pytest.mark.parametrize("fmt", FMTS)
def test_unpack_roundtrip(fmt):
    rng = synth.rng_for(101, fmt, 0)
    for (N, K) in [(5, 1), (7, 333), (64, 4096), (3, 11008)]:
        W = synth.trits(rng, N, K)
        Wp = tri.pack(cuda(W), fmt)
        np.testing.assert_array_equal(host(tri.unpack(Wp, K, fmt)), W)


# ---------------------------------------------------------------- the layer, small and ragged shapes

def run_layer(X, Wp_dev, scale, K, fmt, algo):
    return host(tri.linear(cuda(X), Wp_dev, scale, K, fmt, algo=algo))


def test_small_layer_both_formats_all_algos():
    cfg = configs.SMALL
    for fmt in cfg["fmts"]:
        W, X, s = synth.layer_inputs(cfg["workload_id"], 0, cfg["M"], cfg["N"], cfg["K"], cfg["scale"])
        Wp = tri.pack(cuda(W), fmt)
        for algo in algos_for(cfg["M"], fmt) + [tri.TRI_ALGO_AUTO]:
            say("small layer fmt=%d algo=%d" % (fmt, algo))
            Y = run_layer(X, Wp, s, cfg["K"], fmt, algo)
            worst, exact = check_layer(Y, X, W, s, "small fmt=%d algo=%d" % (fmt, algo))
            say("  worst err/tol %.3g, fraction equal to fp16(ref) %.3f" % (worst, exact))


RAGGED = [(1, 1, 1), (1, 37, 1000), (1, 130, 4097), (1, 300, 81), (1, 33, 12000), (2, 17, 65), (3, 129, 333),
          (5, 300, 81), (16, 50, 4097), (16, 1, 160), (7, 1025, 640), (17, 40, 200), (40, 70, 700),
          (64, 96, 513), (130, 257, 1111), (129, 300, 1000), (200, 513, 2048), (256, 260, 328),
          (150, 100, 64), (96, 600, 320), (33, 700, 1088),
          (13, 4200, 1000), (16, 4111, 2000), (12, 4500, 4096),   # > 256 row blocks of 16 rows
          # workgroups of two and four 16-row blocks (grids of >= 160 such workgroups), ragged ends
          (9, 5200, 2000), (3, 11000, 640), (6, 10250, 1000), (16, 10250, 512), (40, 4100, 1000),
          (33, 5150, 4096),
          # a middling M: the GEMM on quarter-width tiles (at most 64 tiles) and on half-width ones
          (100, 11000, 1000), (300, 16001, 72),
          # long rows: 9..16 steps per wave of eight (2-bit and 1.6-bit), and past that the streaming kernel
          (5, 300, 24000), (16, 200, 30000), (8, 100, 40000), (12, 100, 40000), (20, 90, 26000),
          # two activation rows on the M = 1 kernel's structure (eight and four waves up to 8 steps;
          # sixteen waves for longer 2-bit rows)
          (2, 300, 1000), (2, 4100, 4096), (2, 1000, 11008), (2, 90, 16384), (2, 50, 20000), (2, 300, 30000),
          # wide matrices: the decode kernel with four 16-row blocks per workgroup (2-bit)
          (1, 13000, 1000), (2, 12900, 2048), (1, 14336, 4096),
          # three and four rows on the same structure (2-bit; 1.6-bit takes it only in the block
          # loop over a tall matrix, and the batched kernel elsewhere)
          (3, 300, 1000), (4, 11000, 4096), (4, 4100, 11008), (3, 10300, 2000), (4, 50, 16384)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", RAGGED, ids=["M%dN%dK%d" % s for s in RAGGED])
def test_layer_ragged_shapes(fmt, shape):
    M, N, K = shape
    W, X, s = synth.layer_inputs(200 + fmt, M * 7 + N, M, N, K)
    Wp = tri.pack(cuda(W), fmt)
    for algo in algos_for(M, fmt):
        say("ragged M=%d N=%d K=%d fmt=%d algo=%d" % (M, N, K, fmt, algo))
        check_layer(run_layer(X, Wp, s, K, fmt, algo), X, W, s, "M=%d N=%d K=%d fmt=%d algo=%d" % (M, N, K, fmt, algo))


def test_every_1p6bit_byte_value_in_the_layer():
    """Rows made of all 243 five-trit patterns (each byte value of the 1.6-bit packing once per
    row, in a row-dependent order): every kernel family decodes every byte value."""
    import itertools
    pats = np.array(list(itertools.product((-1, 0, 1), repeat=5)), dtype=np.int8)   # (243, 5)
    N, K = 40, 1280                              # K % 8 == 0: the MFMA decode kernels serve M <= 16
    W = synth.trits(synth.rng_for(231, 0, 0), N, K)
    W[:, :243 * 5] = np.stack([np.roll(pats, 7 * n, axis=0).reshape(-1) for n in range(N)])
    Wp = tri.pack(cuda(W), tri.TRI_FMT_1P6BIT)
    rows = oracle.pack(W, tri.TRI_FMT_1P6BIT)
    assert sorted(set(rows[0][:243].tolist())) == list(range(243))
    for M in (1, 4, 16, 33):
        X = synth.activations(synth.rng_for(230, M, 0), M, K)
        for algo in algos_for(M, tri.TRI_FMT_1P6BIT):
            Y = run_layer(X, Wp, 0.02, K, tri.TRI_FMT_1P6BIT, algo)
            check_layer(Y, X, W, 0.02, "all bytes M=%d algo=%d" % (M, algo))


def test_special_values():
    """Zero weights, all +1 weights, a one-hot activation, a negative scale, fp16 extremes.
    (The scales keep every |Y| below the fp16 range; overflow is covered by test_overflow_to_inf.)"""
    M, N, K = 3, 40, 700
    rng = synth.rng_for(210, 0, 0)
    X = synth.activations(rng, M, K)
    X[1, :5] = [65504, -65504, 6.1e-5, 6e-8, -6e-8]     # largest, smallest normal, subnormals
    X[2] = 0
    X[2, 123] = 1
    for fmt in FMTS:
        for W in (np.zeros((N, K), np.int8), np.ones((N, K), np.int8), synth.trits(rng, N, K)):
            Wp = tri.pack(cuda(W), fmt)
            for algo in algos_for(M, fmt):
                for s in (0.02, -0.375):
                    Y = run_layer(X, Wp, s, K, fmt, algo)
                    check_layer(Y, X, W, s, "special fmt=%d algo=%d" % (fmt, algo))
                    if not W.any():
                        # K % 8 != 0: every kernel serving this shape subtracts the -1 offset as an
                        # exact zero-trit sum, so zero weights give exact zeros.  (The M <= 16
                        # MFMA kernels for K % 8 == 0 subtract sum_k x instead; there W = 0 is
                        # held to the tolerance above.)
                        assert K % 8 != 0 and np.all(Y == 0)
                    # a one-hot activation row returns fp16(scale * t[:, 123]) exactly
                    np.testing.assert_array_equal(Y[2], (np.float32(s) * W[:, 123]).astype(np.float16))


def test_overflow_to_inf():
    """Results beyond the fp16 range round to +-inf (round to nearest even), as the oracle's fp16 rounding does."""
    M, N, K = 2, 64, 256
    X = np.full((M, K), 60000, np.float16)
    X[1] = -1.0
    W = np.ones((N, K), np.int8)
    W[1::2] = -1
    for fmt in FMTS:
        Wp = tri.pack(cuda(W), fmt)
        for algo in algos_for(M, fmt):
            Y = run_layer(X, Wp, 1.0, K, fmt, algo)
            with np.errstate(over="ignore"):
                Yref = oracle.linear_f64(X, W, 1.0).astype(np.float16)
            np.testing.assert_array_equal(Y, Yref)          # +-inf in row 0, exact small values in row 1
            assert np.isinf(Y[0]).all()


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("fmt", FMTS)
def test_invariants(fmt):
    """Deterministic; 2*scale gives 2*Y bitwise (outside the fp16 subnormal range); -X, -W and a
    consistent k permutation stay within tolerance.  (-X does not give -Y bitwise: neither
    v_dot2_f32_f16 nor the MFMA accumulation rounds sign-symmetrically; the fraction is printed.)"""
    import torch
    for (M, N, K) in [(1, 300, 4096), (8, 200, 1000), (40, 130, 700)]:
        W, X, s = synth.layer_inputs(220 + fmt, M, M, N, K)
        Wp = tri.pack(cuda(W), fmt)
        Wn = tri.pack(cuda(-W), fmt)
        Xd = cuda(X)
        for algo in algos_for(M, fmt):
            what = "M=%d N=%d K=%d fmt=%d algo=%d" % (M, N, K, fmt, algo)
            Y1 = host(tri.linear(Xd, Wp, s, K, fmt, algo=algo))
            Y2 = host(tri.linear(Xd, Wp, s, K, fmt, algo=algo))
            np.testing.assert_array_equal(Y1.view(np.uint16), Y2.view(np.uint16), err_msg=what)
            Y2s = host(tri.linear(Xd, Wp, 2 * s, K, fmt, algo=algo))
            normal = np.abs(Y1) >= np.float16(2.0 ** -13)
            np.testing.assert_array_equal(Y2s[normal], 2 * Y1[normal], err_msg=what)
            Yneg = host(tri.linear(-Xd, Wp, s, K, fmt, algo=algo))
            check_layer(Yneg, -X, W, s, "negated X " + what)
            say("%s: -X gives -Y bitwise for %.3f of outputs" % (what, float(np.mean(Yneg == -Y1))))
            check_layer(host(tri.linear(Xd, Wn, s, K, fmt, algo=algo)), X, -W, s, "negated W " + what)
            perm = np.random.default_rng(5).permutation(K)
            Yp = host(tri.linear(cuda(X[:, perm]), tri.pack(cuda(W[:, perm]), fmt), s, K, fmt, algo=algo))
            check_layer(Yp, X, W, s, "k-permuted " + what)
        del Xd
        torch.cuda.synchronize()


def test_misaligned_device_pointer_rejected():
    import torch
    X = torch.zeros(1, 65, dtype=torch.float16, device="cuda")
    Wp = torch.zeros(4, 32, dtype=torch.uint8, device="cuda")
    Y = torch.zeros(1, 4, dtype=torch.float16, device="cuda")
    with pytest.raises(tri.TriError) as e:
        tri.tri_linear(X[:, 1:], Wp, 1.0, 1, 4, 64, F2, Y)
    assert e.value.code == tri.TRI_EALIGN


def test_probe_kernels():
    import torch
    src = torch.arange(1 << 20, dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    tri.tri_probe_copy(src, dst, src.numel() * 4)
    tri.tri_probe_read(src, src.numel() * 4, sink)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


# ---------------------------------------------------------------- the synthetic workloads at full size

@pytest.mark.parametrize("shape", configs.DECODE_SHAPES, ids=[s[0] for s in configs.DECODE_SHAPES])
def test_decode_gemv_full_size(shape):
    name, K, N = shape
    cfg = configs.DECODE
    W, X, s = synth.layer_inputs(cfg["workload_id"], configs.DECODE_SHAPES.index(shape), 1, N, K)
    Wp = tri.pack(cuda(W), F2)
    np.testing.assert_array_equal(host(Wp), oracle.pack2(W))
    for algo in [tri.TRI_ALGO_AUTO] + algos_for(1, F2):
        say("decode %s algo=%d" % (name, algo))
        worst, exact = check_layer(run_layer(X, Wp, s, K, F2, algo), X, W, s, "decode %s algo %d" % (name, algo))
        say("  worst err/tol %.3g, fraction equal to fp16(ref) %.3f" % (worst, exact))


@pytest.mark.parametrize("fmt", FMTS)
def test_batched_decode_full_size(fmt):
    cfg = configs.BATCHED
    for li, (name, K, N) in enumerate(cfg["shapes"]):
        W = synth.trits(synth.rng_for(cfg["workload_id"], li, synth.STREAM_W), N, K)
        Wp = tri.pack(cuda(W), fmt)
        Wp_h = host(Wp)
        np.testing.assert_array_equal(Wp_h, oracle.pack(W, fmt))
        np.testing.assert_array_equal(host(tri.unpack(Wp, K, fmt)), oracle.unpack(Wp_h, K, fmt))
        for M in cfg["Ms"]:
            X = synth.activations(synth.rng_for(cfg["workload_id"], 10 * li + M, synth.STREAM_X), M, K)
            s = synth.uniform_scale(synth.rng_for(cfg["workload_id"], li, synth.STREAM_SCALE))
            say("batched %s M=%d fmt=%d" % (name, M, fmt))
            worst, exact = check_layer(run_layer(X, Wp, s, K, fmt, tri.TRI_ALGO_AUTO), X, W, s,
                                       "batched %s M=%d fmt=%d" % (name, M, fmt))
            say("  worst err/tol %.3g, fraction equal to fp16(ref) %.3f" % (worst, exact))


def test_mid_m_workload_sampled_rows():
    """The middling-M workload as bench.py times it (same inputs, the kernel family tri_linear
    picks): sampled rows, including both sides of every 16-row slice boundary the rows cross."""
    cfg = configs.MID_M
    fmt = cfg["fmt"]
    for li, (name, K, N) in enumerate(cfg["shapes"]):
        for M in cfg["Ms"]:
            W, X, s = synth.layer_inputs(cfg["workload_id"], 10 * li + M, M, N, K)
            rows = sorted({0, 1, 15, 16, 17, M // 2, M - 17, M - 16, M - 1})
            say("mid-M %s M=%d algo=%s" % (name, M, tri.ALGO_NAMES[tri.tri_select_algo(M, N, K, fmt)]))
            Y = run_layer(X, tri.pack(cuda(W), fmt), s, K, fmt, tri.TRI_ALGO_AUTO)
            worst, exact = check_layer(Y, X, W, s, "mid-M %s M=%d" % (name, M), rows=rows)
            say("  worst err/tol %.3g, fraction equal to fp16(ref) %.3f" % (worst, exact))


@pytest.mark.parametrize("M", configs.BLOCK["Ms"])
def test_block_step(M):
    """Seven chained linears of one decode block with the glue on the CPU: every GPU linear is
    checked on the input the oracle chain gives it, and the GPU chain's output against the
    oracle chain's."""
    cfg = configs.BLOCK
    layers = {}
    for li, (name, K, N) in enumerate(cfg["layers"]):
        W = synth.trits(synth.rng_for(cfg["workload_id"], li, synth.STREAM_W), N, K)
        s = synth.uniform_scale(synth.rng_for(cfg["workload_id"], li, synth.STREAM_SCALE))
        layers[name] = (W, tri.pack(cuda(W), cfg["fmt"]), s, K)
    x0 = synth.activations(synth.rng_for(cfg["workload_id"], 100 + M, synth.STREAM_X), M, cfg["hidden"])

    def gpu_linear(name, a):
        W, Wp, s, K = layers[name]
        return run_layer(a, Wp, s, K, cfg["fmt"], tri.TRI_ALGO_AUTO)

    def ref_linear(name, a):
        W, _, s, _ = layers[name]
        return oracle.linear_f64(a, W, s).astype(np.float16)

    say("block step M=%d" % M)
    out_ref, ins_ref = block_glue.block_step(x0, ref_linear)
    for name, a in ins_ref.items():
        W, _, s, _ = layers[name]
        check_layer(gpu_linear(name, a), a, W, s, "block M=%d layer %s" % (M, name))
    out_gpu, _ = block_glue.block_step(x0, gpu_linear)
    rel = np.linalg.norm(out_gpu - out_ref) / np.linalg.norm(out_ref)
    say("  block output relative difference GPU chain vs oracle chain: %.3g" % rel)
    assert rel < 1e-2


# Whole 128-row tiles of the prefill GEMM: the first row band (every 32-row MFMA sub-tile of
# every column tile, including those of the half-width tail launch at N = 28672) and the last.
PREFILL_ROWS = list(range(0, 128)) + list(range(1920, 2048))


@pytest.mark.parametrize("li", [0, 1])
def test_prefill_full_size_whole_tiles(li):
    """M = 2048 on both prefill shapes and both formats: the oracle's reference for the rows of two
    whole 128-row tiles is computed once and every output element of those rows is checked."""
    import torch
    cfg = configs.PREFILL
    name, K, N = cfg["shapes"][li]
    M = cfg["M"]
    say("prefill %s: generating inputs" % name)
    W = synth.trits(synth.rng_for(cfg["workload_id"], li, synth.STREAM_W), N, K)
    X = synth.activations(synth.rng_for(cfg["workload_id"], li, synth.STREAM_X), M, K)
    s = cfg["scale"]
    say("prefill %s: oracle on %d rows" % (name, len(PREFILL_ROWS)))
    Xs = X[PREFILL_ROWS]
    Yref = oracle.linear_f64(Xs, W, s)
    tol = oracle.tolerance(Xs, s, Yref)
    Xd = cuda(X)
    for fmt in cfg["fmts"]:
        Wd = cuda(W)
        Wp = tri.pack(Wd, fmt)
        del Wd
        say("prefill %s fmt=%d: pack check" % (name, fmt))
        np.testing.assert_array_equal(host(Wp), oracle.pack(W, fmt))
        say("prefill %s fmt=%d: linear" % (name, fmt))
        Y = host(tri.linear(Xd, Wp, s, K, fmt))
        assert np.all(np.isfinite(Y))
        err = np.abs(Y[PREFILL_ROWS].astype(np.float64) - Yref)
        bad = int((err > tol).sum())
        worst = float((err / tol).max())
        say("  worst err/tol %.3g, out of tolerance %d" % (worst, bad))
        assert bad == 0, "prefill %s fmt=%d: %d elements out of tolerance (worst err/tol %.3g)" % (name, fmt, bad, worst)
        del Wp
        torch.cuda.empty_cache()


# Full-width GEMM tiles (128 x 512) with ragged edges in M and N and an odd number of K tiles:
# 8 x 32 = 256 tiles, so no half-width tail launch; sampled rows cover every 32-row MFMA sub-tile
# of the first row tile (rows 32..95 with 0, 1, 127) and the last partial tile.
GEMM_EDGE_ROWS = [0, 1] + list(range(32, 96)) + [127, 128, 500, 895, 896, 997, 998, 999]


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_full_tiles_ragged_edges(fmt):
    M, N, K = 1000, 16000, 328
    W, X, s = synth.layer_inputs(300 + fmt, 1, M, N, K)
    Wp = tri.pack(cuda(W), fmt)
    say("gemm full tiles M=%d N=%d K=%d fmt=%d" % (M, N, K, fmt))
    Y = run_layer(X, Wp, s, K, fmt, tri.TRI_ALGO_GEMM)
    assert np.all(np.isfinite(Y))
    worst, exact = check_layer(Y, X, W, s, "gemm edges fmt=%d" % fmt, rows=GEMM_EDGE_ROWS)
    say("  worst err/tol %.3g, fraction equal to fp16(ref) %.3f" % (worst, exact))


# Grouped layers: several matrices reading the same activations, one launch where the small-M
# kernels serve every matrix (K = 1000: the grouped kernels, also over 16-row slices for M > 16;
# K = 1001: one launch per matrix).
GROUPED = [(1, 1000), (2, 1000), (3, 1000), (16, 1000), (1, 1001), (5, 1001), (20, 1000), (40, 1000), (20, 1001)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("case", GROUPED, ids=["M%dK%d" % c for c in GROUPED])
def test_grouped_layers(fmt, case):
    import torch
    M, K = case
    Ns = [37, 256, 100]
    X = synth.activations(synth.rng_for(400 + fmt, M, synth.STREAM_X), M, K)
    Ws = [synth.trits(synth.rng_for(400 + fmt, 10 * M + g, synth.STREAM_W), n, K) for g, n in enumerate(Ns)]
    scales = [0.02, -0.03, 0.045]
    Xd = cuda(X)
    Wps = [tri.pack(cuda(W), fmt) for W in Ws]
    Ys = [torch.empty((M, n), dtype=torch.float16, device="cuda") for n in Ns]
    say("grouped M=%d K=%d fmt=%d" % (M, K, fmt))
    tri.tri_linear_grouped(Xd, Wps, scales, M, Ns, K, fmt, Ys)
    for g, (W, s, Y) in enumerate(zip(Ws, scales, Ys)):
        Yh = host(Y)
        check_layer(Yh, X, W, s, "grouped M=%d K=%d fmt=%d g=%d" % (M, K, fmt, g))
        # the same kernels as a single layer: identical results
        np.testing.assert_array_equal(Yh, host(tri.linear(Xd, Wps[g], s, K, fmt)))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 2, 4, 8, 16, 24])
def test_grouped_large_grid_same_as_single(fmt, M):
    """Q, K, V-like projections (3 x 4096 rows; 3 x 8192 at M <= 2): the grouped grid is large
    enough for workgroups of several 16-row blocks while each single layer's is not; the results
    are bitwise the same."""
    import torch
    K = 1000
    Ns = [8192, 8192, 8192] if M <= 2 else [4096, 4096, 4096]
    X = synth.activations(synth.rng_for(410 + fmt, M, synth.STREAM_X), M, K)
    Ws = [synth.trits(synth.rng_for(410 + fmt, 10 * M + g, synth.STREAM_W), n, K) for g, n in enumerate(Ns)]
    scales = [0.02, -0.03, 0.045]
    Xd = cuda(X)
    Wps = [tri.pack(cuda(W), fmt) for W in Ws]
    Ys = [torch.empty((M, n), dtype=torch.float16, device="cuda") for n in Ns]
    say("grouped 3x4096 M=%d K=%d fmt=%d" % (M, K, fmt))
    tri.tri_linear_grouped(Xd, Wps, scales, M, Ns, K, fmt, Ys)
    for g, (W, s, Y) in enumerate(zip(Ws, scales, Ys)):
        Yh = host(Y)
        check_layer(Yh, X, W, s, "grouped 3x4096 M=%d fmt=%d g=%d" % (M, fmt, g))
        np.testing.assert_array_equal(Yh, host(tri.linear(Xd, Wps[g], s, K, fmt)))


# Tall single matrices, where the decode kernel runs a resident grid whose workgroups loop over
# the 16-row blocks (at least two blocks per resident workgroup); the last has more than sixteen
# blocks per workgroup, so its outputs are written out in several rounds.
TALL = [(tri.TRI_FMT_2BIT, 1, 40007, 4096), (tri.TRI_FMT_2BIT, 2, 40007, 4096),
        (tri.TRI_FMT_2BIT, 1, 30011, 8192), (tri.TRI_FMT_1P6BIT, 1, 40003, 4096),
        (tri.TRI_FMT_1P6BIT, 2, 40003, 8192), (tri.TRI_FMT_2BIT, 1, 212005, 512),
        (tri.TRI_FMT_2BIT, 2, 212005, 512), (tri.TRI_FMT_2BIT, 3, 30011, 8192), (tri.TRI_FMT_2BIT, 4, 40007, 4096),
        (tri.TRI_FMT_1P6BIT, 3, 30011, 8192), (tri.TRI_FMT_1P6BIT, 4, 40003, 4096),
        # the largest staged-operand instances of the loop: four rows over six (2-bit) and five
        # (1.6-bit) steps per wave, 563 blocks against 512 resident workgroups
        (tri.TRI_FMT_2BIT, 4, 9000, 11008), (tri.TRI_FMT_1P6BIT, 4, 9000, 12000),
        # one 2-bit row of 8192 < K <= 16384: the loop on sixteen waves of three and four steps
        (tri.TRI_FMT_2BIT, 1, 40007, 11008), (tri.TRI_FMT_2BIT, 1, 20011, 16384)]


@pytest.mark.parametrize("fmt,M,N,K", TALL)
def test_block_loop_tall_matrices(fmt, M, N, K):
    """Every output against the oracle, and bitwise against the same matrix launched in a group
    (whose grid has one workgroup per block) where the group takes the same kernel: up to two
    rows, and four for 2-bit (1.6-bit groups of three or four rows take the batched kernel)."""
    import torch
    W, X, s = synth.layer_inputs(520 + fmt, N % 1000 + M, M, N, K)
    W2 = synth.trits(synth.rng_for(520 + fmt, 7, synth.STREAM_W), 64, K)
    Xd = cuda(X)
    Wp, Wp2 = tri.pack(cuda(W), fmt), tri.pack(cuda(W2), fmt)
    say("tall M=%d N=%d K=%d fmt=%d" % (M, N, K, fmt))
    Y = host(tri.linear(Xd, Wp, s, K, fmt))
    worst, exact = check_layer(Y, X, W, s, "tall M=%d N=%d K=%d fmt=%d" % (M, N, K, fmt))
    say("  worst err/tol %.3g, fraction equal to fp16(ref) %.3f" % (worst, exact))
    if M <= 2 or fmt == tri.TRI_FMT_2BIT:
        Ys = [torch.empty((M, N), dtype=torch.float16, device="cuda"),
              torch.empty((M, 64), dtype=torch.float16, device="cuda")]
        tri.tri_linear_grouped(Xd, [Wp, Wp2], [s, 0.03], M, [N, 64], K, fmt, Ys)
        np.testing.assert_array_equal(Y, host(Ys[0]))


def test_grouped_tall_matrices_same_as_single():
    """Two tall 2-bit matrices (at least three 16-row blocks per resident sixteen-wave workgroup) of
    rows between 8192 and 16384 trits at one activation row: alone each runs the sixteen-wave block
    loop, together the sixteen-wave one-shot grid; the outputs are the oracle's within the bound and
    bitwise the same either way."""
    import torch
    M, K, Ns = 1, 11008, [12300, 12400]
    X = synth.activations(synth.rng_for(530, 1, synth.STREAM_X), M, K)
    Ws = [synth.trits(synth.rng_for(530, 10 + g, synth.STREAM_W), n, K) for g, n in enumerate(Ns)]
    scales = [0.02, -0.035]
    Xd = cuda(X)
    Wps = [tri.pack(cuda(W), F2) for W in Ws]
    Ys = [torch.empty((M, n), dtype=torch.float16, device="cuda") for n in Ns]
    say("grouped tall 2 x ~12300 rows K=%d" % K)
    tri.tri_linear_grouped(Xd, Wps, scales, M, Ns, K, F2, Ys)
    for g, (W, s, Y) in enumerate(zip(Ws, scales, Ys)):
        Yh = host(Y)
        check_layer(Yh, X, W, s, "grouped tall g=%d" % g)
        np.testing.assert_array_equal(Yh, host(tri.linear(Xd, Wps[g], s, K, F2)))


# 2-bit tiles of 5..8 rows over rows of 8192 < K <= 12288 trits run on sixteen waves when the matrix
# alone takes one 16-row block per workgroup; the choice is per matrix, so a group of such matrices
# is one sixteen-wave launch and a mixed group one launch per matrix.
# (1.6-bit: twelve waves, rows of 10240 < K <= 15360 trits.)
WIDE16 = [(F2, 8, 11008, [4096, 3000]), (F2, 5, 9000, [4096, 3000]), (F2, 8, 11008, [4096, 6000]),
          (F2, 6, 9000, [6000, 4096]), (F16, 8, 11008, [4096, 3000]), (F16, 7, 14000, [6000, 4096]),
          (F16, 4, 11008, [4096, 3000]), (F16, 3, 14000, [6000, 4096])]


@pytest.mark.parametrize("fmt,M,K,Ns", WIDE16,
                         ids=["f%dM%dK%d_%d_%d" % (c[0], c[1], c[2], c[3][0], c[3][1]) for c in WIDE16])
def test_grouped_wide_rows_same_as_single(fmt, M, K, Ns):
    """Every output against the oracle, and bitwise against the same matrix launched alone, for
    groups whose matrices all take the wide (sixteen- or twelve-wave) variant and for mixed groups."""
    import torch
    X = synth.activations(synth.rng_for(540, M, synth.STREAM_X), M, K)
    Ws = [synth.trits(synth.rng_for(540, 10 * M + g + Ns[g] % 97, synth.STREAM_W), n, K) for g, n in enumerate(Ns)]
    scales = [0.025, -0.04]
    Xd = cuda(X)
    Wps = [tri.pack(cuda(W), fmt) for W in Ws]
    Ys = [torch.empty((M, n), dtype=torch.float16, device="cuda") for n in Ns]
    say("grouped wide rows fmt=%d M=%d K=%d Ns=%s" % (fmt, M, K, Ns))
    tri.tri_linear_grouped(Xd, Wps, scales, M, Ns, K, fmt, Ys)
    for g, (W, s, Y) in enumerate(zip(Ws, scales, Ys)):
        Yh = host(Y)
        check_layer(Yh, X, W, s, "grouped wide rows fmt=%d M=%d K=%d g=%d" % (fmt, M, K, g))
        np.testing.assert_array_equal(Yh, host(tri.linear(Xd, Wps[g], s, K, fmt)))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [4, 8, 16])
def test_grouped_three_blocks_same_as_single(fmt, M):
    """A group of 4096 and 7000 rows takes three 16-row blocks per workgroup (232 workgroups, one
    round) while the 4096-row matrix alone takes one: the block count changes no arithmetic, so the
    outputs are the oracle's within the bound and bitwise the same either way."""
    import torch
    K, Ns = 1000, [4096, 7000]
    X = synth.activations(synth.rng_for(550 + fmt, M, synth.STREAM_X), M, K)
    Ws = [synth.trits(synth.rng_for(550 + fmt, 10 * M + g, synth.STREAM_W), n, K) for g, n in enumerate(Ns)]
    scales = [0.02, -0.03]
    Xd = cuda(X)
    Wps = [tri.pack(cuda(W), fmt) for W in Ws]
    Ys = [torch.empty((M, n), dtype=torch.float16, device="cuda") for n in Ns]
    say("grouped three blocks M=%d fmt=%d" % (M, fmt))
    tri.tri_linear_grouped(Xd, Wps, scales, M, Ns, K, fmt, Ys)
    for g, (W, s, Y) in enumerate(zip(Ws, scales, Ys)):
        check_layer(host(Y), X, W, s, "grouped three blocks M=%d fmt=%d g=%d" % (M, fmt, g))
    np.testing.assert_array_equal(host(Ys[0]), host(tri.linear(Xd, Wps[0], scales[0], K, fmt)))
