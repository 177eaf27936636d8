"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these checks re-types the oracle's own formulas: the packings are
checked against Python's base-3 / base-4 positional parsing (int(s, base) and
numpy.base_repr), the fp16 decoder against numpy's float16, and the layer
against exact integer arithmetic, numpy's float64 matmul on tiny shapes and
textbook special cases.  Page facts come from tests/golden/packing_facts.json,
each with its citation.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from bit_mixed_precision_tri_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))
FACTS = json.load(open(os.path.join(HERE, "golden", "packing_facts.json")))

F2, F16 = oracle.FMT_2BIT, oracle.FMT_1P6BIT


def all_patterns(k):
    """All 3^k ternary patterns of length k, as a (3^k, k) int8 matrix (itertools order)."""
    import itertools
    return np.array(list(itertools.product((-1, 0, 1), repeat=k)), dtype=np.int8)


def digits_to_int(row, base):
    """Positional value of the digits (t+1), lowest index least significant, by int(str, base)."""
    s = "".join(str(int(t) + 1) for t in reversed(row))
    return int(s, base)


# ---------------------------------------------------------------- P1: closed forms

def test_lossless_condition_and_density():
    k, p = FACTS["trits_per_byte_1p6"]["value"], FACTS["bits_per_byte"]["value"]
    assert 2 ** p > 3 ** k                       # 256 > 243
    assert 2 ** (p - 1) < 3 ** k                 # 7 bits are not enough
    assert p / k == FACTS["bits_per_weight_1p6"]["value"]
    # minimal p for k trits is ceil(k log2 3); 2^p > 3^k holds strictly from there on
    for kk in range(1, 16):
        pmin = math.ceil(kk * math.log2(3))
        assert 2 ** pmin > 3 ** kk and 2 ** (pmin - 1) < 3 ** kk
    assert round(math.log2(3), FACTS["information_limit_bits"]["digits"]) == FACTS["information_limit_bits"]["value"]
    assert FACTS["radix_2bit"]["value"] ** 4 == 2 ** 8 and 3 <= FACTS["radix_2bit"]["value"]


@pytest.mark.parametrize("K", [64, 80, 320, 4096 * 5 // 4, 64 * 80])
def test_oracle_density_matches_page_bits_per_weight(K):
    if K % 64 == 0:
        assert oracle.row_bytes(K, F2) * 8 / K == FACTS["bits_per_weight_2bit"]["value"]
    if K % 80 == 0:
        assert oracle.row_bytes(K, F16) * 8 / K == FACTS["bits_per_weight_1p6"]["value"]


def test_row_bytes_at_workload_shapes_and_eightfold_saving():
    # 16*ceil(K/64) and 16*ceil(K/80) evaluated by hand for the workload K values
    expect2 = {512: 128, 4096: 1024, 11008: 2752, 8192: 2048, 28672: 7168}
    expect16 = {512: 112, 4096: 832, 11008: 2208, 8192: 1648, 28672: 5744}
    for K in expect2:
        assert oracle.row_bytes(K, F2) == expect2[K]
        assert oracle.row_bytes(K, F16) == expect16[K]
        assert 2 * K / oracle.row_bytes(K, F2) == FACTS["memory_reduction_vs_16bit"]["value"]
        # 1.6-bit padding to 16-byte rows costs at most 15 bytes over ceil(K/5)
        assert 0 <= oracle.row_bytes(K, F16) - math.ceil(K / 5) <= 15
    assert oracle.row_bytes(0, F2) == -1 and oracle.row_bytes(5, 7) == -1


# ---------------------------------------------------------------- P2: exhaustive patterns

def test_pack16_all_243_patterns_is_base3_bijection():
    P = all_patterns(5)
    packed = oracle.pack16(P)                    # K = 5: one data byte + 15 pad bytes per row
    first = packed[:, 0].astype(int)
    assert sorted(first.tolist()) == list(range(243))          # bijection onto 0..242
    for row, b in zip(P, first):
        assert b == digits_to_int(row, 3)
    assert np.all(packed[:, 1:] == digits_to_int([0] * 5, 3))  # padding = five zero trits
    np.testing.assert_array_equal(oracle.unpack(packed, 5, F16), P)


def test_pack2_all_81_patterns_is_base4_bijection():
    P = all_patterns(4)
    packed = oracle.pack2(P)
    first = packed[:, 0].astype(int)
    assert len(set(first.tolist())) == 81
    for row, b in zip(P, first):
        assert b == digits_to_int(row, 4)
        assert all(((b >> (2 * j)) & 3) != 3 for j in range(4))   # code 3 never emitted
    assert np.all(packed[:, 1:] == digits_to_int([0] * 4, 4))
    np.testing.assert_array_equal(oracle.unpack(packed, 4, F2), P)


# ---------------------------------------------------------------- P3: every byte value

def test_unpack_every_byte_value():
    Wp2 = np.zeros((256, oracle.row_bytes(4, F2)), np.uint8)
    Wp2[:, 0] = np.arange(256)
    Wp16 = np.zeros((256, oracle.row_bytes(5, F16)), np.uint8)
    Wp16[:, 0] = np.arange(256)
    U2 = oracle.unpack(Wp2, 4, F2)
    U16 = oracle.unpack(Wp16, 5, F16)
    for b in range(256):
        d4 = [int(c) for c in reversed(np.base_repr(b, 4).zfill(4))]
        assert U2[b].tolist() == [0 if d == 3 else d - 1 for d in d4]
        d3 = [int(c) for c in reversed(np.base_repr(b, 3).zfill(6))][:5]   # 6 digits only for b >= 243
        assert U16[b].tolist() == [d - 1 for d in d3]


# ---------------------------------------------------------------- theorem: unpack(pack(W)) = W

@pytest.mark.parametrize("fmt", [F2, F16])
def test_roundtrip_all_residues(fmt):
    rng = synth.rng_for(900, fmt, 0)
    for K in list(range(1, 170)) + [4095, 4096, 4097, 11008]:
        W = synth.trits(rng, 3, K)
        Wp = oracle.pack(W, fmt)
        assert Wp.shape == (3, oracle.row_bytes(K, fmt))
        np.testing.assert_array_equal(oracle.unpack(Wp, K, fmt), W)
        # everything beyond K decodes to zero trits
        Kp = Wp.shape[1] * (4 if fmt == F2 else 5)
        full = oracle.unpack(Wp, Kp, fmt)
        assert np.all(full[:, K:] == 0)


def test_pack_encodes_sign_of_any_int8():
    W = np.array([[-128, -5, -1, 0, 1, 7, 127, 0, 3, -3]], dtype=np.int8)
    for fmt in (F2, F16):
        np.testing.assert_array_equal(oracle.unpack(oracle.pack(W, fmt), W.shape[1], fmt), np.sign(W))


# ---------------------------------------------------------------- fp16 decoding

def test_half_decoder_all_65536_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# ---------------------------------------------------------------- P5: exact-sum invariant

def exact_sums(X, W):
    """sum_k t*x exactly: every finite fp16 is an integer multiple of 2^-24 below 2^16."""
    xi = (X.astype(np.float64) * 2.0 ** 24).astype(np.int64)       # exact, |xi| < 2^40
    assert np.array_equal(xi.astype(np.float64) * 2.0 ** -24, X.astype(np.float64))
    return [[sum(int(t) * int(x) for t, x in zip(W[n], xi[m])) for n in range(W.shape[0])]
            for m in range(X.shape[0])]


def test_exact_sum_invariant():
    rng = synth.rng_for(901, 0, 0)
    for (M, N, K) in [(2, 5, 97), (1, 3, 4096), (3, 2, 1000)]:
        W = synth.trits(rng, N, K)
        # wide dynamic range, including fp16 subnormals and large values
        X = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-26, 12, (M, K)))).astype(np.float16)
        X[np.isinf(X)] = 0
        Y = oracle.linear_f64(X, W, 1.0)
        S = exact_sums(X, W)
        for m in range(M):
            for n in range(N):
                assert Y[m, n] == S[m][n] * 2.0 ** -24          # bit-exact
        Y4 = oracle.linear_f64(X, W, 0.25)                      # power-of-two scale is exact too
        assert np.array_equal(Y4, Y * 0.25)


# ---------------------------------------------------------------- P6: brute force on tiny shapes

def test_tiny_shapes_match_numpy_matmul():
    rng = synth.rng_for(902, 0, 0)
    for M in (1, 2, 3):
        for N in (1, 4, 7):
            for K in range(1, 14):
                W = synth.trits(rng, N, K)
                X = synth.activations(rng, M, K)
                s = synth.uniform_scale(rng)
                ref = s * (X.astype(np.float64) @ W.astype(np.float64).T)   # exact sums -> same bits
                np.testing.assert_array_equal(oracle.linear_f64(X, W, s), ref)
                for fmt in (F2, F16):
                    np.testing.assert_array_equal(
                        oracle.linear_packed_f64(X, oracle.pack(W, fmt), K, fmt, s), ref)


# ---------------------------------------------------------------- P7: special cases

def test_special_cases():
    rng = synth.rng_for(903, 0, 0)
    M, N, K = 3, 6, 37
    X = synth.activations(rng, M, K)
    x64 = X.astype(np.float64)
    s = 0.03125
    assert np.all(oracle.linear_f64(X, np.zeros((N, K), np.int8), s) == 0)
    ones = np.ones((N, K), np.int8)
    np.testing.assert_array_equal(oracle.linear_f64(X, ones, s), np.repeat(s * x64.sum(1, keepdims=True), N, 1))
    for j in (0, 17, K - 1):
        for sign in (1, -1):
            E = np.zeros((1, K), np.int8)
            E[0, j] = sign
            np.testing.assert_array_equal(oracle.linear_f64(X, E, s)[:, 0], sign * s * x64[:, j])
    W = synth.trits(rng, N, K)
    for k in (0, 5, K - 1):
        Xe = np.zeros((1, K), np.float16)
        Xe[0, k] = 1
        np.testing.assert_array_equal(oracle.linear_f64(Xe, W, s)[0], s * W[:, k].astype(np.float64))
    W1 = synth.trits(rng, N, 1)
    np.testing.assert_array_equal(oracle.linear_f64(X[:, :1], W1, s), s * x64[:, :1] @ W1.T.astype(np.float64))


# ---------------------------------------------------------------- P8/P9: invariants

def test_sign_symmetry_and_k_permutation_invariance():
    rng = synth.rng_for(904, 0, 0)
    M, N, K = 4, 9, 333
    W = synth.trits(rng, N, K)
    X = synth.activations(rng, M, K)
    s = 0.02
    Y = oracle.linear_f64(X, W, s)
    assert np.array_equal(oracle.linear_f64(X, -W, s), -Y)
    assert np.array_equal(oracle.linear_f64(-X, W, s), -Y)
    assert np.array_equal(oracle.linear_f64(X, W, -s), -Y)
    perm = rng.permutation(K)
    assert np.array_equal(oracle.linear_f64(X[:, perm], W[:, perm], s), Y)   # exact sums: order-free


def test_rows_are_independent_and_thread_count_does_not_matter():
    rng = synth.rng_for(905, 0, 0)
    W = synth.trits(rng, 50, 300)
    X = synth.activations(rng, 3, 300)
    Y = oracle.linear_f64(X, W, 0.02, nthreads=1)
    assert np.array_equal(oracle.linear_f64(X, W, 0.02, nthreads=4), Y)
    assert np.array_equal(oracle.linear_f64(X[1:2], W[7:9], 0.02), Y[1:2, 7:9])


def test_nonfinite_activation_rejected():
    X = np.zeros((1, 8), np.float16)
    X[0, 3] = np.inf
    with pytest.raises(ValueError):
        oracle.linear_f64(X, np.ones((2, 8), np.int8), 1.0)
    X[0, 3] = np.nan
    with pytest.raises(ValueError):
        oracle.linear_f64(X, np.ones((2, 8), np.int8), 1.0)


def test_tolerance_formula_shape():
    X = np.array([[1, -2, 0.5]], np.float16)
    Yref = np.array([[10.0, -4.0]])
    tol = oracle.tolerance(X, -0.5, Yref)
    np.testing.assert_allclose(tol, [[2e-3 * 0.5 * 3.5 + 1e-2, 2e-3 * 0.5 * 3.5 + 4e-3]])


# ---------------------------------------------------------------- quantiser (latent weights -> trits + scale)
# Pins: hand-worked ties and clipping, exact recovery of a scaled ternary matrix, the scale against
# numpy's mean (a library routine summing in another order), power-of-two and sign invariance, the
# degenerate cases, and the zero fraction of Gaussian weights against its closed form.

def test_quantize_worked_ties_and_clipping():
    # sum |w| = 4 over 4 weights, so the scale is exactly 1 and w / scale = w:
    #   0.5 + 2^-20 -> 1 (above the midpoint);  0.5 -> 0 (a tie goes to the even neighbour 0);
    #   -(0.5 - 2^-20) -> 0;  2.5 -> round 2, clipped to 1
    T, s = oracle.quantize(np.array([[0.5 + 2.0 ** -20, 0.5, -(0.5 - 2.0 ** -20), 2.5]], np.float32))
    assert s == np.float32(1.0)
    np.testing.assert_array_equal(T, [[1, 0, 0, 1]])
    #   -0.5 -> 0 (tie);  -1.5 -> -2 (tie to even), clipped to -1;  1 -> 1;  1 -> 1
    T, s = oracle.quantize(np.array([[-0.5, -1.5, 1.0, 1.0]], np.float32))
    assert s == np.float32(1.0)
    np.testing.assert_array_equal(T, [[0, -1, 1, 1]])
    # two rows: sum |w| = 0.75 + 0.25 + 0.5 + 0.5 = 2 over 4 weights, scale 0.5;
    # w / scale = 1.5 -> 1 (clipped from 2), 0.5 -> 0 (tie), -1 -> -1, 1 -> 1
    T, s = oracle.quantize(np.array([[0.75, 0.25], [-0.5, 0.5]], np.float32))
    assert s == np.float32(0.5)
    np.testing.assert_array_equal(T, [[1, 0], [-1, 1]])


@pytest.mark.parametrize("c", [0.0123, 3.5, 1e-3, 7.0e-6])
def test_quantize_recovers_scaled_ternary(c):
    from fractions import Fraction
    rng = synth.rng_for(950, 0, 0)
    Tin = synth.trits(rng, 23, 157)
    c32 = np.float32(c)
    W = Tin.astype(np.float32) * c32                   # exact: entries are 0 and +-c32
    T, s = oracle.quantize(W)
    np.testing.assert_array_equal(T, Tin)            # |w| / scale = N*K / nnz >= 1 for nonzeros
    exact = Fraction(float(c32)) * int(np.count_nonzero(Tin)) / Tin.size
    assert abs(Fraction(float(s)) - exact) <= Fraction(float(np.spacing(s)))


def test_quantize_scale_is_the_mean_absolute_value():
    rng = synth.rng_for(951, 0, 0)
    for (N, K, std) in [(37, 301, 0.02), (5, 4096, 1.0), (300, 7, 3e-4)]:
        W = (rng.standard_normal((N, K)) * std).astype(np.float32)
        _, s = oracle.quantize(W)
        ref = np.float32(np.mean(np.abs(W.astype(np.float64))))
        assert abs(float(s) - float(ref)) <= float(np.spacing(ref)), (N, K, s, ref)


def test_quantize_power_of_two_and_sign_invariance():
    rng = synth.rng_for(952, 0, 0)
    W = (rng.standard_normal((19, 211)) * 0.05).astype(np.float32)
    T, s = oracle.quantize(W)
    for e in (-7, 5):
        T2, s2 = oracle.quantize(W * np.float32(2.0 ** e))
        np.testing.assert_array_equal(T2, T)
        assert s2 == s * np.float32(2.0 ** e)
    Tn, sn = oracle.quantize(-W)
    np.testing.assert_array_equal(Tn, -T)
    assert sn == s


def test_quantize_degenerate_cases():
    T, s = oracle.quantize(np.zeros((3, 5), np.float32))
    assert s == 0 and not T.any()
    T, s = oracle.quantize(np.array([[-3.0]], np.float32))
    assert s == np.float32(3.0) and T[0, 0] == -1
    # one subnormal among many zeros: the mean underflows to a zero scale, and a zero scale gives zero trits
    W = np.zeros((64, 64), np.float32)
    W[3, 4] = np.float32(1.4e-45)
    T, s = oracle.quantize(W)
    assert s == 0 and not T.any()
    for bad in (np.inf, -np.inf, np.nan):
        W = np.ones((2, 3), np.float32)
        W[1, 2] = bad
        with pytest.raises(ValueError):
            oracle.quantize(W)


def test_quantize_zero_fraction_of_gaussian_weights():
    # For w ~ N(0, sigma^2) the scale tends to E|w| = sigma*sqrt(2/pi), and a weight rounds to 0 when
    # |w| < scale/2, which has probability erf(sqrt(2/pi)/2/sqrt(2)) = erf(1/(2*sqrt(pi))) ~ 0.3103.
    rng = synth.rng_for(953, 0, 0)
    W = (rng.standard_normal((1000, 1000)) * 0.02).astype(np.float32)
    T, s = oracle.quantize(W)
    p0 = math.erf(0.5 / math.sqrt(math.pi))
    assert abs(np.mean(T == 0) - p0) < 3e-3
    assert abs(np.mean(T == 1) - (1 - p0) / 2) < 3e-3
    assert abs(float(s) - 0.02 * math.sqrt(2.0 / math.pi)) < 1e-4


# ---------------------------------------------------------------- the layer with block glue folded around it
# With W the identity (t[n][k] = 1 if n == k) and scale 1, Y is the layer's effective input itself,
# so the glue can be checked against closed forms without re-typing it.

def identity(K):
    return np.eye(K, dtype=np.int8)


def test_fused_without_glue_is_the_plain_layer():
    rng = synth.rng_for(970, 0, 0)
    W = synth.trits(rng, 11, 97)
    X = synth.activations(rng, 3, 97)
    np.testing.assert_array_equal(oracle.linear_fused_f64(X, W, 0.02), oracle.linear_f64(X, W, 0.02))


def test_fused_rmsnorm_normalises_rows():
    rng = synth.rng_for(971, 0, 0)
    K = 64
    X = synth.activations(rng, 4, K)
    Y = oracle.linear_fused_f64(X, identity(K), 1.0, norm=True, eps=0.0)
    np.testing.assert_allclose(np.mean(Y * Y, axis=1), 1.0, rtol=1e-12)            # unit mean square
    ratio = Y / X.astype(np.float64)                                              # a positive factor per row
    assert np.all(ratio > 0)
    np.testing.assert_allclose(ratio, ratio[:, :1] * np.ones((1, K)), rtol=1e-12)
    # a constant row c: x / sqrt(c^2 + eps)
    Xc = np.full((1, K), 0.5, np.float16)
    Yc = oracle.linear_fused_f64(Xc, identity(K), 1.0, norm=True, eps=0.25)
    np.testing.assert_allclose(Yc, 0.5 / math.sqrt(0.25 + 0.25), rtol=1e-15)
    # a power-of-two rescaling of the input changes nothing (eps = 0)
    np.testing.assert_array_equal(oracle.linear_fused_f64(X * np.float16(4), identity(K), 1.0, norm=True, eps=0.0), Y)
    # the gain multiplies feature k
    gain = np.linspace(-2, 2, K).astype(np.float16)
    Yg = oracle.linear_fused_f64(X, identity(K), 1.0, norm=True, eps=0.0, gain=gain)
    np.testing.assert_allclose(Yg, Y * gain.astype(np.float64), rtol=1e-15, atol=1e-300)


def test_silu_closed_forms():
    z = np.array([0.0, math.log(3.0), -math.log(3.0), 2.0, -2.0, 30.0, -30.0])
    out = oracle.silu_mul_f64(z, np.ones_like(z))
    assert out[0] == 0.0                                                       # silu(0) = 0
    assert abs(out[1] - 0.75 * math.log(3.0)) < 1e-15                          # sigmoid(ln 3) = 3/4
    assert abs((out[1] - out[2]) - math.log(3.0)) < 1e-15                      # silu(z) - silu(-z) = z
    assert abs((out[3] - out[4]) - 2.0) < 1e-15
    assert abs(out[5] - 30.0) < 1e-11 and abs(out[6]) < 1e-11                  # silu(z) -> max(z, 0)
    b = np.array([1.0, -2.0, 0.5, 3.0, 3.0, 1.0, 1.0])
    np.testing.assert_allclose(oracle.silu_mul_f64(z, b), out * b, rtol=1e-15)   # the gate scales b


def test_silu_pair_with_identity_weights():
    # gate and up layers both the identity: the output is silu(x) * x
    z = np.array([[0.0, math.log(3.0), -math.log(3.0), 2.0]], np.float16)
    z64 = z.astype(np.float64)[0]
    out = oracle.silu_pair_f64(z, identity(4), 1.0, identity(4), 1.0)[0]
    assert out[0] == 0.0
    np.testing.assert_allclose(out[1], z64[1] * z64[1] / (1 + math.exp(-z64[1])), rtol=1e-15)
    assert abs(out[1] - 0.75 * z64[1] ** 2) < 2e-3
    # a gate scale of 0 gives silu(0) = 0 everywhere
    assert not oracle.silu_pair_f64(z, identity(4), 0.0, identity(4), 1.0).any()
    # the up scale multiplies the output
    np.testing.assert_allclose(oracle.silu_pair_f64(z, identity(4), 1.0, identity(4), -3.0)[0], -3.0 * out,
                               rtol=1e-15)
    # normalised inputs: both layers see the same unit-mean-square activations
    X = synth.activations(synth.rng_for(973, 0, 0), 2, 64)
    n = oracle.linear_fused_f64(X, identity(64), 1.0, norm=True, eps=0.0)
    np.testing.assert_allclose(oracle.silu_pair_f64(X, identity(64), 1.0, identity(64), 1.0, norm=True, eps=0.0),
                               n / (1 + np.exp(-n)) * n, rtol=1e-14)


def test_fused_residual_and_nonfinite_inputs():
    rng = synth.rng_for(972, 0, 0)
    M, N, K = 2, 5, 40
    X = synth.activations(rng, M, K)
    R = synth.activations(rng, M, N)
    # zero weights leave exactly the residual
    np.testing.assert_array_equal(oracle.linear_fused_f64(X, np.zeros((N, K), np.int8), 0.7, residual=R),
                                  R.astype(np.float64))
    # the residual adds to the scaled product
    W = synth.trits(rng, N, K)
    np.testing.assert_allclose(oracle.linear_fused_f64(X, W, 0.7, residual=R),
                               oracle.linear_f64(X, W, 0.7) + R.astype(np.float64), rtol=1e-15, atol=1e-15)
    for kw in (dict(residual=np.full((M, N), np.inf, np.float16)), dict(norm=True, gain=np.full(K, np.nan, np.float16))):
        with pytest.raises(ValueError):
            oracle.linear_fused_f64(X, W, 0.7, **kw)
