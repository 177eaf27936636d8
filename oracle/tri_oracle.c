/*
 * tri_oracle.c -- CPU ORACLE for the ternary linear layer.  TEST INFRASTRUCTURE ONLY.
 *
 * This is the plain, slow, obviously-correct reference that the HIP library is
 * checked against.  It is not part of the product: only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark load it.  It shares no
 * source, header, table or helper with the HIP library, and the HIP library never
 * loads it.
 *
 * What it follows (the web pages on Spectra 1.1, arXiv 2506.23025):
 *   [PR] "Pith review of Spectra 1.1: Scaling Laws and Efficient Inference for
 *        Ternary Language Models" (pith.science):
 *        - "What carries the argument": a ternary linear layer has a weight matrix
 *          in {-1,0,1} times one shared floating-point scale; k trits fit
 *          losslessly in p bits when 2^p > 3^k, so k=5 trits fit in p=8 bits
 *          (1.6 bits per weight).
 *        - "Core claim": lossless 2-bit packing by base-4 encoding and 1.6-bit
 *          packing by base-3 encoding.
 *        - "Referee Report", minor comment 5 (paper section 3.2): the 1.6-bit
 *          decode is written as a sequence b'_i -> x_i; the final partial block is
 *          not specified.
 *        - "Significance": the packing correctness theorem (paper Appendix E),
 *          i.e. unpacking a packed block returns the block.
 *   [SP] "Spectra 1.1: Scaling Laws and Efficient Inference for Ternary Language
 *        Models" (shd-paper.top summary), abstract: 2-bit and 1.6-bit packing of
 *        ternary weights.
 *   For the quantiser, [PR] "What carries the argument" (latent full-precision
 *   weights rounded on the fly in the forward pass) and the review's list of
 *   domain assumptions (round-to-nearest ternary quantisation, straight-through
 *   estimation).
 *
 * Readings taken where the pages are silent (stated once here, used below):
 *   - digit of a trit t is d = t + 1 in {0,1,2} (non-negative base-4 / base-3 digits);
 *   - the lowest k index is the least-significant digit of its byte;
 *   - a row of K trits is padded with zero trits (d = 1) to a multiple of 64 trits
 *     (2-bit, 16 bytes) or 80 trits (1.6-bit, 16 bytes); rows are stored one after
 *     another, output row n first (out x in, like nn.Linear);
 *   - packing encodes sign(w), so any int8 input is accepted;
 *   - unpack is defined for every byte value: 2-bit code 3 gives 0; 1.6-bit bytes
 *     243..255 go through the same repeated division by 3;
 *   - the layer returns scale * sum_k t[n][k] * x[m][k] exactly as summed in
 *     float64 in k order, unrounded;
 *   - the block glue folded around a layer (the pages name the block's parts, not
 *     their placement): RMSNorm of the input before the product, the residual added
 *     to the scaled sum, the SiLU gate applied to two layers' unrounded outputs, all
 *     in float64;
 *   - the quantiser's scale (the pages do not give its rule) is the mean absolute
 *     value of the matrix, summed in float64 and rounded once to float32; a weight
 *     becomes round-half-to-even(w / scale) clipped to [-1, 1], and a zero scale
 *     gives zero trits.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC tri_oracle.c -o liboracle.so
 */
#include <stdint.h>
#include <stddef.h>
#include <math.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_FMT_2BIT = 0, OR_FMT_1P6BIT = 1 };

/* Bytes of one packed row: 16*ceil(K/64) for 2-bit, 16*ceil(K/80) for 1.6-bit; -1 if invalid. */
int64_t oracle_row_bytes(int64_t K, int fmt)
{
    if (K < 1) return -1;
    if (fmt == OR_FMT_2BIT) return 16 * ((K + 63) / 64);
    if (fmt == OR_FMT_1P6BIT) return 16 * ((K + 79) / 80);
    return -1;
}

/* Digit of weight w: sign(w) + 1. */
static int digit_of(int8_t w)
{
    if (w > 0) return 2;
    if (w < 0) return 0;
    return 1;
}

/* Trit k of row n, zero beyond the end of the row. */
static int8_t trit_at(const int8_t *W, int64_t K, int64_t n, int64_t k)
{
    if (k >= K) return 0;
    return W[n * K + k];
}

/* 2-bit packing, base-4 encoding ([PR] "Core claim"):
 * byte b of row n = sum_{j=0..3} d(4b+j) * 4^j. */
void oracle_pack2(const int8_t *W, int64_t N, int64_t K, uint8_t *Wp)
{
    int64_t S = oracle_row_bytes(K, OR_FMT_2BIT);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < S; ++b) {
            int value = 0;
            int power = 1;
            for (int j = 0; j < 4; ++j) {
                value += digit_of(trit_at(W, K, n, 4 * b + j)) * power;
                power *= 4;
            }
            Wp[n * S + b] = (uint8_t)value;
        }
    }
}

/* 1.6-bit packing, base-3 encoding of 5 trits per byte, possible because
 * 3^5 = 243 < 2^8 ([PR] "What carries the argument", "Core claim"):
 * byte b of row n = sum_{j=0..4} d(5b+j) * 3^j, evaluated by Horner's rule. */
void oracle_pack16(const int8_t *W, int64_t N, int64_t K, uint8_t *Wp)
{
    int64_t S = oracle_row_bytes(K, OR_FMT_1P6BIT);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < S; ++b) {
            int value = 0;
            for (int j = 4; j >= 0; --j)
                value = value * 3 + digit_of(trit_at(W, K, n, 5 * b + j));
            Wp[n * S + b] = (uint8_t)value;
        }
    }
}

/* Unpack (inverse of the two packings; [PR] "Significance", Appendix E theorem;
 * "Referee Report" minor comment 5 for the b'_i -> x_i iteration).
 * Writes the first K trits of every row. Returns 0, or -1 on an unknown format. */
int oracle_unpack(const uint8_t *Wp, int64_t N, int64_t K, int fmt, int8_t *W)
{
    int64_t S = oracle_row_bytes(K, fmt);
    if (S < 0) return -1;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < S; ++b) {
            int byte = Wp[n * S + b];
            if (fmt == OR_FMT_2BIT) {
                for (int j = 0; j < 4; ++j) {
                    int64_t k = 4 * b + j;
                    int code = (byte >> (2 * j)) & 3;
                    int t = (code == 3) ? 0 : code - 1;
                    if (k < K) W[n * K + k] = (int8_t)t;
                }
            } else {
                int rest = byte;                 /* b'_0 */
                for (int j = 0; j < 5; ++j) {
                    int x = rest % 3;            /* x_j = b'_j mod 3 */
                    rest = rest / 3;             /* b'_{j+1} = floor(b'_j / 3) */
                    int64_t k = 5 * b + j;
                    if (k < K) W[n * K + k] = (int8_t)(x - 1);
                }
            }
        }
    }
    return 0;
}

/* IEEE 754 binary16 bit pattern -> double (exact). */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int exponent = (h >> 10) & 0x1f;
    int mantissa = h & 0x3ff;
    double v;
    if (exponent == 0)
        v = ldexp((double)mantissa, -24);               /* subnormal or zero */
    else if (exponent == 31)
        v = mantissa ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + mantissa), exponent - 25);
    return sign ? -v : v;
}

/* The ternary linear layer ([PR] "What carries the argument"):
 *   Y[m][n] = scale * sum_{k<K} t[n][k] * x[m][k]
 * X holds M*K fp16 bit patterns (row-major), W holds N*K trits (row-major),
 * Y receives M*N float64 values, unrounded.  Sums run over k in order, in float64.
 * Returns 0, or -1 if X holds a non-finite value (the layer is defined on finite
 * activations only).  nthreads > 0 sets the OpenMP thread count (output rows are
 * split between threads; each element keeps its own k order, so the result does
 * not depend on it). */
int oracle_linear_f64(const uint16_t *X, const int8_t *W, double scale,
                      int64_t M, int64_t N, int64_t K, double *Y, int nthreads)
{
    for (int64_t i = 0; i < M * K; ++i)
        if (!isfinite(oracle_half_to_double(X[i]))) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    for (int64_t m = 0; m < M; ++m) {
        #pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            double sum = 0.0;
            for (int64_t k = 0; k < K; ++k)
                sum += (double)W[n * K + k] * oracle_half_to_double(X[m * K + k]);
            Y[m * N + n] = scale * sum;
        }
    }
    return 0;
}

/* Ternary quantisation of latent full-precision weights ([PR] "What carries the
 * argument": the layer's weights are latent full-precision values rounded on the
 * fly to {-1,0,1} times one shared scale; the review's domain assumptions name the
 * rounding as round-to-nearest).  The scale rule is a reading (see the header):
 *   scale = (sum_n sum_k |w[n][k]|) / (N*K), each row summed in k order, the row
 *           sums added in n order, all in float64, then rounded to float32;
 *   t[n][k] = clip(round_half_even(w[n][k] / scale), -1, 1), or 0 when scale == 0.
 * W is N*K float32 row-major; T receives N*K trits.  Returns 0, or -1 if W holds a
 * non-finite value. */
int oracle_quantize(const float *W, int64_t N, int64_t K, int8_t *T, float *scale)
{
    for (int64_t i = 0; i < N * K; ++i)
        if (!isfinite(W[i])) return -1;
    double total = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        double row = 0.0;
        for (int64_t k = 0; k < K; ++k)
            row += fabs((double)W[n * K + k]);
        total += row;
    }
    float s = (float)(total / ((double)N * (double)K));
    *scale = s;
    for (int64_t i = 0; i < N * K; ++i) {
        double q = 0.0;
        if (s != 0.0f) {
            q = rint((double)W[i] / (double)s);    /* nearest, ties to even (default rounding mode) */
            if (q > 1.0) q = 1.0;
            if (q < -1.0) q = -1.0;
        }
        T[i] = (int8_t)q;
    }
    return 0;
}

/* The ternary linear layer with the glue of a decode block folded around it
 * ([PR] "If this is right": the end-to-end speed-up falls short of the layer's
 * because of the work outside the linear layers).  For activation row m, in float64
 * and unrounded:
 *   x2[k] = norm ? x[m][k] * gain[k] / sqrt(mean_k(x[m][k]^2) + eps) : x[m][k]
 *           (gain NULL: a gain of 1);
 *   Y[m][n] = (residual ? residual[m][n] : 0) + scale * sum_k t[n][k] * x2[k].
 * X: M*K fp16 bit patterns; gain: K fp16 bit patterns; residual: M*N fp16 bit
 * patterns; W: N*K trits; Y: M*N float64.  Returns 0, or -1 on a non-finite input. */
int oracle_linear_fused_f64(const uint16_t *X, int norm, const uint16_t *gain, double eps,
                            const int8_t *W, double scale, const uint16_t *residual,
                            int64_t M, int64_t N, int64_t K, double *Y)
{
    for (int64_t i = 0; i < M * K; ++i)
        if (!isfinite(oracle_half_to_double(X[i]))) return -1;
    for (int64_t k = 0; gain && k < K; ++k)
        if (!isfinite(oracle_half_to_double(gain[k]))) return -1;
    for (int64_t i = 0; residual && i < M * N; ++i)
        if (!isfinite(oracle_half_to_double(residual[i]))) return -1;
    double *x = (double *)malloc((size_t)K * sizeof(double));
    if (!x) return -1;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k) x[k] = oracle_half_to_double(X[m * K + k]);
        if (norm) {
            double sq = 0.0;
            for (int64_t k = 0; k < K; ++k) sq += x[k] * x[k];
            double r = sqrt(sq / (double)K + eps);
            for (int64_t k = 0; k < K; ++k)
                x[k] = x[k] * (gain ? oracle_half_to_double(gain[k]) : 1.0) / r;
        }
        for (int64_t n = 0; n < N; ++n) {
            double sum = 0.0;
            for (int64_t k = 0; k < K; ++k) sum += (double)W[n * K + k] * x[k];
            Y[m * N + n] = (residual ? oracle_half_to_double(residual[m * N + n]) : 0.0) + scale * sum;
        }
    }
    free(x);
    return 0;
}

/* The SiLU gate of a gated MLP applied to two layer outputs: out[i] = silu(a[i]) * b[i],
 * silu(z) = z / (1 + exp(-z)), in float64. */
void oracle_silu_mul_f64(const double *a, const double *b, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = a[i] / (1.0 + exp(-a[i])) * b[i];
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
