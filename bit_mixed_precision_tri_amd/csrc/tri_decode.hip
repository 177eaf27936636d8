// tri_decode.hip -- ternary linear layer for a few activation rows (1 <= M <= 16) on MFMA.
//
// The layer (Pith review of "Spectra 1.1", "What carries the argument"):
//   Y[m][n] = scale * sum_k t[n][k] * X[m][k],  t in {-1, 0, +1},  fp32 accumulation.
// The contraction runs on v_mfma_f32_16x16x32_f16 with the trits decoded in registers
// (M padded to the 16 rows of the instruction); the review names the pages' GPU kernel an
// FP16 x INT2 tensor-core kernel with fused dequantisation, which this replaces on gfx950.
//
// Decode.  Masking a packed register leaves each trit's digit d = t + 1 in the low bits
// of an fp16 half, which reads exactly as d * 4^p * 2^-24 (p = the digit's position in its
// 16-bit half).  The MFMA B operand is the 16-byte weight chunk itself, masked as a whole:
// one v_and_or_b32 per register, no repacking.  One MFMA only mixes trits of one position,
// so it accumulates exact products into a per-position-class accumulator, and the classes
// are merged with exact powers of two.  Since t = d - 1, the sums of zero trits (d = 1) are
// subtracted: column 15 of every B operand is a row of zero trits instead of a weight row
// (15 weight rows per block) -- its lanes read nothing and OR in the bytes of one -- so
// the same instruction produces the correction with the same arithmetic, and for an
// all-zero weight row the difference is exactly zero.  1.6-bit bytes first go through a
// 256-entry LDS table to the 2-bit digit layout (five base-3 digits: the repeated division
// b'_i -> x_i that the review's referee report describes for the paper's section 3.2).
//
// Data flow.  A workgroup of NW waves owns one block of 15 weight rows; the waves split
// its 16-byte chunks (K split): lane (g = lane/16, j = lane%16) of wave w reads chunk
// 4*(s*NW + w) + g of row j at chunk-step s, so one buffer load reads 64 contiguous bytes of
// 15 rows.  Every weight chunk of the wave is requested at the start; reads past the
// matrix return zero (buffer range check) and chunks past the row end meet zero
// activations.  The activations are loaded once per workgroup, permuted into the MFMA
// A-operand order (a 2-bit register pairs trits (16w+p, 16w+8+p), a 1.6-bit one trits
// (5q+p, 5q+40+p); the sum over k is order-free) and staged in LDS, GS chunk-steps at a
// time.  The waves' partial tiles are summed through LDS in a fixed order (no atomics).
#include "tri_device.h"
#include "tri_internal.h"

namespace tri {

constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer resource, gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

__device__ __forceinline__ u32x4 buffer_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
}

__device__ __forceinline__ float4_t mfma(const u32x4 a, const u32x4 b, float4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c, 0,
                                                  0, 0);
}

template <int FMT, int MT, int NW, int CST, int GS>
__global__ __launch_bounds__(64 * NW) void k_decode(const uint16_t *__restrict__ X, const uint8_t *__restrict__ Wp,
                                                    float scale, int M, int N, int K, int C,
                                                    uint16_t *__restrict__ Y)
{
    constexpr bool TWO = FMT == TRI_FMT_2BIT;
    constexpr int NPOS = TWO ? 8 : 10;           // MFMAs (A operands) per 16-byte chunk
    constexpr int NCLS = TWO ? 6 : 5;            // position classes
    constexpr int XH = TWO ? 64 : 80;            // activations per chunk
    constexpr int GCH = 4 * NW * GS;             // chunks staged per group
    constexpr int NG = CST / GS;                 // groups
    constexpr int IPT = (GCH * MT + 64 * NW - 1) / (64 * NW);   // staging items per thread
    static_assert(CST % GS == 0, "groups must tile the chunk-steps");
    __shared__ u32x4 xa[GCH * NPOS * MT];        // [chunk][operand][activation row]
    __shared__ uint32_t lut[TWO ? 1 : 256];
    __shared__ float red[NW][MT][16];

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int j = lane & 15;
    const int n0 = blockIdx.x * 15;
    const int64_t S = (int64_t)C * 16;
    const int items = GCH * M;                   // (chunk, activation row) pairs per group

    if constexpr (!TWO) {
        for (int b = threadIdx.x; b < 256; b += 64 * NW) lut[b] = base3_digits_2bit((uint32_t)b);
    }

    // (1) activations of group 0 (buffer reads; pieces past the row end are forced out of range)
    const __amdgpu_buffer_rsrc_t xr_rsrc = buffer_rsrc(X, (uint32_t)((int64_t)M * K * 2));
    u32x4 xr[IPT][XH / 8];
    auto load_group = [&](int gi) {
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int item = it * 64 * NW + threadIdx.x;
            const int cl = item / M, i = item - cl * M;
            const int k0 = (gi * GCH + cl) * XH;
            const uint32_t base = (uint32_t)(i * K + k0) * 2u;
#pragma unroll
            for (int q = 0; q < XH / 8; ++q) {
                const bool in = item < items && k0 + 8 * q < K;
                xr[it][q] = buffer_ld16(xr_rsrc, in ? base + 16u * q : 0x80000000u, 0);
            }
        }
    };
    load_group(0);

    // (2) every weight chunk of this wave.  Rows past N and bytes past the matrix read as
    //     zero; lanes j = 15 read nothing and later OR in the zero-trit digits.
    const int rows_here = min(15, N - n0);
    const __amdgpu_buffer_rsrc_t w_rsrc = buffer_rsrc(Wp + n0 * S, (uint32_t)(rows_here * S));
    const uint32_t wbase = j < 15 ? (uint32_t)(j * S + (4 * wv + g) * 16) : 0x80000000u;
    u32x4 wq[CST];
#pragma unroll
    for (int s = 0; s < CST; ++s) wq[s] = buffer_ld16(w_rsrc, wbase + (uint32_t)(s * 64 * NW), 0);

    // the zero-trit column: its lanes read zeros; OR-ing in the bytes of a zero-trit row
    // (digits 1: 0x55 for 2-bit, 121 for 1.6-bit) makes the usual decode produce its digits
    const uint32_t zfill = j == 15 ? (TWO ? 0x55555555u : 0x79797979u) : 0u;
    // A rows >= M only feed tile rows that are never stored: any staged row will do
    const int arow = min(j, M - 1);

    const float4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    float4_t acc[NCLS];
#pragma unroll
    for (int c = 0; c < NCLS; ++c) acc[c] = zero4;

#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        if (gi > 0) {
            __syncthreads();                     // group gi-1 is no longer read
            load_group(gi);
        }
        // (3) stage the A operands of (chunk, row) items
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int item = it * 64 * NW + threadIdx.x;
            if (item < items) {
                const int cl = item / M, i = item - cl * M;
                u32x4 *dst = xa + (cl * NPOS) * MT + i;
                uint32_t x32[XH / 2];
#pragma unroll
                for (int q = 0; q < XH / 8; ++q) {
                    x32[4 * q] = xr[it][q][0]; x32[4 * q + 1] = xr[it][q][1];
                    x32[4 * q + 2] = xr[it][q][2]; x32[4 * q + 3] = xr[it][q][3];
                }
                if constexpr (TWO) {
#pragma unroll
                    for (int p = 0; p < 8; ++p) {
                        u32x4 a;
#pragma unroll
                        for (int w = 0; w < 4; ++w)
                            a[w] = (p & 1) ? pair_halves<1>(x32[8 * w + 4 + p / 2], x32[8 * w + p / 2])
                                           : pair_halves<0>(x32[8 * w + 4 + p / 2], x32[8 * w + p / 2]);
                        dst[p * MT] = a;
                    }
                } else {
#pragma unroll
                    for (int p = 0; p < 5; ++p)
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            u32x4 a;
#pragma unroll
                            for (int qq = 0; qq < 4; ++qq) {
                                const int e = 5 * (4 * h + qq) + p;
                                a[qq] = (e & 1) ? pair_halves<1>(x32[(e >> 1) + 20], x32[e >> 1])
                                                : pair_halves<0>(x32[(e >> 1) + 20], x32[e >> 1]);
                            }
                            dst[(2 * p + h) * MT] = a;
                        }
                }
            }
        }
        __syncthreads();

        // (4) the chunk-steps of this group
#pragma unroll
        for (int sl = 0; sl < GS; ++sl) {
            const int s = gi * GS + sl;
            if (4 * (s * NW + wv) >= C) break;   // wave-uniform: no chunk of this step is live
            const u32x4 *asrc = xa + (4 * (sl * NW + wv) + g) * NPOS * MT + arow;
            const u32x4 v = wq[s] | zfill;
            if constexpr (TWO) {
                const u32x4 u = v >> 12u;
#pragma unroll
                for (int p = 0; p < 6; ++p) acc[p] = mfma(asrc[p * MT], v & (0x00030003u << (2 * p)), acc[p]);
                acc[0] = mfma(asrc[6 * MT], u & 0x00030003u, acc[0]);
                acc[1] = mfma(asrc[7 * MT], u & 0x000C000Cu, acc[1]);
            } else {
                u32x4 lo, hi;                    // bytes q (lo) and q+8 (hi) of the chunk, as digit codes
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const uint32_t blo = (v[q >> 2] >> (8 * (q & 3))) & 0xFFu;
                    const uint32_t bhi = (v[2 + (q >> 2)] >> (8 * (q & 3))) & 0xFFu;
                    const uint32_t pq = lut[blo] | (lut[bhi] << 16);
                    if (q < 4) lo[q] = pq; else hi[q - 4] = pq;
                }
#pragma unroll
                for (int p = 0; p < 5; ++p) {
                    const uint32_t m = 0x00030003u << (2 * p);
                    acc[p] = mfma(asrc[(2 * p) * MT], lo & m, acc[p]);
                    acc[p] = mfma(asrc[(2 * p + 1) * MT], hi & m, acc[p]);
                }
            }
        }
    }

    // (5) merge the classes with exact powers of two, sum the waves' tiles in a fixed order,
    //     subtract column 15 (the zero-trit sums) and undo the 2^-24 of the decoded digits
    float4_t t = acc[0] + 0.25f * acc[1];
    t += 0.0625f * acc[2] + 0.015625f * acc[3];
    t += 0.00390625f * acc[4];
    if constexpr (TWO) t += 0.0009765625f * acc[5];
#pragma unroll
    for (int v = 0; v < 4; ++v)
        if (4 * g + v < MT) red[wv][4 * g + v][j] = t[v];   // lane (g, j): tile rows 4g..4g+3, column j
    __syncthreads();
    for (int idx = threadIdx.x; idx < M * 15; idx += 64 * NW) {
        const int i = idx / 15, jj = idx - i * 15;
        if (n0 + jj < N) {
            float sw = 0.f, sz = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                sw += red[w][i][jj];
                sz += red[w][i][15];
            }
            Y[(int64_t)i * N + n0 + jj] = __builtin_bit_cast(uint16_t, (_Float16)(((sw - sz) * 16777216.0f) * scale));
        }
    }
}

// M = 1 variant: every wave stages only the activation chunks it will use, in its own LDS
// region, so no wave waits for another before computing.  Lane l < 4*CST of wave w loads
// the 64 (80) activations of chunk c(s, g) = 4*(s*NW + w) + g with l = 4s + g, permutes
// them into the A-operand order and writes them; after that only the final tile reduction
// synchronises the workgroup.  A rows 1..15 (lanes j > 0) read the same staged row: their
// tile rows are never stored.
template <int FMT, int MT, int NW, int CST, int GS>
static void launch_dec(const uint16_t *X, const uint8_t *Wp, float scale, int M, int N, int K, int C, uint16_t *Y,
                       hipStream_t s)
{
    hipLaunchKernelGGL((k_decode<FMT, MT, NW, CST, GS>), dim3((N + 14) / 15), dim3(64 * NW), 0, s, X, Wp, scale, M, N,
                       K, C, Y);
}

// 2 <= M <= 16 with short rows: activations staged per workgroup, a few chunk-steps at a time.
// (Longer rows go to the streaming small-M kernel, which measured faster there.)
template <int FMT>
static bool launch_mn(const uint16_t *X, const uint8_t *Wp, float scale, int M, int N, int K, int C, uint16_t *Y,
                      hipStream_t s)
{
    if (C > 64) return false;
    if (M <= 4) launch_dec<FMT, 4, 4, 4, 4>(X, Wp, scale, M, N, K, C, Y, s);
    else if (FMT == TRI_FMT_1P6BIT) launch_dec<FMT, 16, 2, 8, 1>(X, Wp, scale, M, N, K, C, Y, s);
    else launch_dec<FMT, 16, 4, 4, 1>(X, Wp, scale, M, N, K, C, Y, s);
    return true;
}

bool launch_decode(const uint16_t *X, const uint8_t *Wp, float scale, int M, int N, int K, int fmt, uint16_t *Y,
                   hipStream_t s)
{
    const int C = (int)(row_bytes(K, fmt) / 16);
    // 32-bit buffer offsets: the activations and one 15-row block must stay below 2^31 bytes;
    // the activation pieces are 8 values wide, so K must be a multiple of 8
    if ((K % 8) != 0 || (int64_t)M * K * 2 >= ((int64_t)1 << 31) || 15 * (int64_t)C * 16 >= ((int64_t)1 << 31))
        return false;
    const Groups gr = make_groups(1, &Wp, &scale, &N, &Y);
    if (M == 1) return launch_mv1(X, gr, K, fmt, s);
    if (M <= 4 && launch_mvr(X, gr, M, K, fmt, s)) return true;
    if (launch_mvm(X, gr, M, K, fmt, s)) return true;
    return fmt == TRI_FMT_2BIT ? launch_mn<TRI_FMT_2BIT>(X, Wp, scale, M, N, K, C, Y, s)
                               : launch_mn<TRI_FMT_1P6BIT>(X, Wp, scale, M, N, K, C, Y, s);
}

}  // namespace tri
