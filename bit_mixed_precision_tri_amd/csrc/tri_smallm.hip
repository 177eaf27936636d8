// tri_smallm.hip -- ternary linear layer for a few activation rows (1 <= M <= 16) on MFMA.
//
// The layer (Pith review of "Spectra 1.1", "What carries the argument"):
//   Y[m][n] = scale * sum_k t[n][k] * X[m][k],  t in {-1, 0, +1},  fp32 accumulation.
// The review describes the pages' GPU kernel as an FP16 x INT2 tensor-core kernel with
// fused dequantisation ("What carries the argument"); here the contraction runs on
// gfx950's v_mfma_f32_16x16x32_f16 with the trits decoded in registers, and M is padded
// to the 16 rows of the instruction (rows >= M carry zeros).
//
// Decode into MFMA operands.  The B operand of one MFMA holds, per lane, 8 fp16 values:
// here 4 registers, each a pair of trits masked out of a packed word in place.  The mask
// leaves the digit d = t + 1 of each trit in the low bits of an fp16 half, which reads as
// d * 4^p * 2^-24 exactly (p = the digit's position inside its 16-bit half; fp16
// subnormals, or the lowest exponent bits for p = 5).  One MFMA only ever mixes trits of
// the same position p, so it accumulates sum d*x*4^p*2^-24 exactly-multiplied in fp32, into
// one accumulator per position class.  The -1 of t = d - 1 becomes one extra MFMA per
// activation fragment whose B holds the digits of zero trits (d = 1) at the same
// position; it runs in the same order into its own class accumulators, shared by all row
// blocks of the wave, and is subtracted class by class (exactly cancelling all-zero
// weights).  Then the classes are merged with exact powers of two.
//   2-bit:   word bits 2p / 16+2p hold trits (16w+p, 16w+8+p); positions 6, 7 are taken
//            from the word shifted right by 12, so they share the classes of 0, 1.
//   1.6-bit: each packed byte is first mapped through a 256-entry LDS table to its five
//            base-3 digits at bits 2j (the repeated division b'_i -> x_i of the paper's
//            section 3.2 as described in the review's referee report, tabulated); bytes
//            q and q+8 of a 16-byte chunk share a register, so position p yields the trit
//            pair (5q+p, 5q+40+p).
// The sum over k is order-free, so the activations are permuted (v_perm_b32) into the
// same pairing instead of reshuffling the weights.
//
// Work split.  A wave owns R blocks of 16 weight rows; lane (g = lane/16, j = lane%16)
// loads 16-byte chunk (4*wave + g) + 4*NW*i of row j of every block, so each load
// instruction reads 64 contiguous bytes of 16 rows.  The NW waves of a workgroup split
// the chunks of the same rows; their partial tiles are summed through LDS in a fixed
// order (no atomics).
#include "tri_device.h"
#include "tri_internal.h"

namespace tri {

template <int FMT, int R, int NW>
__global__ __launch_bounds__(64 * NW) void k_smallm(const uint16_t *__restrict__ X, const uint8_t *__restrict__ Wp,
                                                    float scale, int M, int N, int K, int C,
                                                    uint16_t *__restrict__ Y)
{
    constexpr bool TWO = FMT == TRI_FMT_2BIT;
    constexpr int NCLS = TWO ? 6 : 5;            // position classes
    constexpr int XH = TWO ? 64 : 80;            // activations per 16-byte chunk
    __shared__ uint32_t lut[TWO ? 1 : 256];
    __shared__ float red[NW > 1 ? NW : 1][R][256];

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int j = lane & 15;
    const int n0 = blockIdx.x * 16 * R;
    const int64_t S = (int64_t)C * 16;

    if (!TWO) {
        for (int b = threadIdx.x; b < 256; b += 64 * NW) lut[b] = base3_digits_2bit((uint32_t)b);
        __syncthreads();
    }

    const float4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    float4_t acc[R][NCLS];
    float4_t accz[NCLS];                                 // class sums of zero trits (digit 1)
#pragma unroll
    for (int c = 0; c < NCLS; ++c) accz[c] = zero4;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < NCLS; ++c) acc[r][c] = zero4;

    const bool xrow_live = j < M;                       // A row i = j of this lane
    const uint16_t *xrow = X + (int64_t)(xrow_live ? j : 0) * K;
    const bool xvec = (K % 8) == 0;

    for (int c0 = 4 * wv; c0 < C; c0 += 4 * NW) {      // wave-uniform trip count
        const int c = c0 + g;
        const bool live = c < C;
        uint4 wq[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = min(n0 + 16 * r + j, N - 1);   // rows past N repeat the last; never stored
            wq[r] = live ? ld16(Wp + row * S + (int64_t)c * 16) : make_uint4(0, 0, 0, 0);
        }
        uint32_t xr[XH / 2];
        if (live && xrow_live) {
            load_x_span<XH>(xrow, c * XH, K, xvec, xr);
        } else {
#pragma unroll
            for (int q = 0; q < XH / 2; ++q) xr[q] = 0u;
        }
        if constexpr (TWO) {
            // A fragment of position p: (x[16w+p], x[16w+8+p]) for w = 0..3
            uint32_t xa[8][4];
#pragma unroll
            for (int w = 0; w < 4; ++w)
#pragma unroll
                for (int p = 0; p < 8; p += 2) {
                    xa[p][w] = pair_halves<0>(xr[8 * w + 4 + p / 2], xr[8 * w + p / 2]);
                    xa[p + 1][w] = pair_halves<1>(xr[8 * w + 4 + p / 2], xr[8 * w + p / 2]);
                }
#pragma unroll
            for (int p = 0; p < 6; ++p) {
                const uint32_t z = 0x00010001u << (2 * p);
                accz[p] = mfma16(xa[p][0], xa[p][1], xa[p][2], xa[p][3], z, z, z, z, accz[p]);
            }
            accz[0] = mfma16(xa[6][0], xa[6][1], xa[6][2], xa[6][3], 0x00010001u, 0x00010001u, 0x00010001u,
                             0x00010001u, accz[0]);
            accz[1] = mfma16(xa[7][0], xa[7][1], xa[7][2], xa[7][3], 0x00040004u, 0x00040004u, 0x00040004u,
                             0x00040004u, accz[1]);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t v[4] = {wq[r].x, wq[r].y, wq[r].z, wq[r].w};
                const uint32_t u[4] = {v[0] >> 12, v[1] >> 12, v[2] >> 12, v[3] >> 12};
#pragma unroll
                for (int p = 0; p < 6; ++p) {
                    const uint32_t m = 0x00030003u << (2 * p);
                    acc[r][p] = mfma16(xa[p][0], xa[p][1], xa[p][2], xa[p][3], v[0] & m, v[1] & m, v[2] & m, v[3] & m,
                                       acc[r][p]);
                }
                acc[r][0] = mfma16(xa[6][0], xa[6][1], xa[6][2], xa[6][3], u[0] & 0x00030003u, u[1] & 0x00030003u,
                                   u[2] & 0x00030003u, u[3] & 0x00030003u, acc[r][0]);
                acc[r][1] = mfma16(xa[7][0], xa[7][1], xa[7][2], xa[7][3], u[0] & 0x000C000Cu, u[1] & 0x000C000Cu,
                                   u[2] & 0x000C000Cu, u[3] & 0x000C000Cu, acc[r][1]);
            }
        } else {
            // A fragment of (position p, half h): (x[5q+p], x[5q+40+p]) for q = 4h..4h+3
            uint32_t xa[5][8];
#pragma unroll
            for (int q = 0; q < 8; ++q)
#pragma unroll
                for (int p = 0; p < 5; ++p) {
                    const int e = 5 * q + p;
                    xa[p][q] = (e & 1) ? pair_halves<1>(xr[(e >> 1) + 20], xr[e >> 1])
                                       : pair_halves<0>(xr[(e >> 1) + 20], xr[e >> 1]);
                }
#pragma unroll
            for (int p = 0; p < 5; ++p) {
                const uint32_t z = 0x00010001u << (2 * p);
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    accz[p] = mfma16(xa[p][4 * h], xa[p][4 * h + 1], xa[p][4 * h + 2], xa[p][4 * h + 3], z, z, z, z,
                                     accz[p]);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t wd[4] = {wq[r].x, wq[r].y, wq[r].z, wq[r].w};
                uint32_t pq[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const uint32_t blo = (wd[q >> 2] >> (8 * (q & 3))) & 0xFFu;          // byte q
                    const uint32_t bhi = (wd[2 + (q >> 2)] >> (8 * (q & 3))) & 0xFFu;    // byte q+8
                    pq[q] = lut[blo] | (lut[bhi] << 16);
                }
#pragma unroll
                for (int p = 0; p < 5; ++p) {
                    const uint32_t m = 0x00030003u << (2 * p);
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        acc[r][p] = mfma16(xa[p][4 * h], xa[p][4 * h + 1], xa[p][4 * h + 2], xa[p][4 * h + 3],
                                           pq[4 * h] & m, pq[4 * h + 1] & m, pq[4 * h + 2] & m, pq[4 * h + 3] & m,
                                           acc[r][p]);
                }
            }
        }
    }

    // Subtract the zero-trit class sums, merge the classes (exact power-of-two weights),
    // undo the 2^-24 of the decoded digits, and combine the waves.
    float res[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float4_t t = (acc[r][0] - accz[0]) + 0.25f * (acc[r][1] - accz[1]);
        t += 0.0625f * (acc[r][2] - accz[2]) + 0.015625f * (acc[r][3] - accz[3]);
        t += 0.00390625f * (acc[r][4] - accz[4]);
        if constexpr (TWO) t += 0.0009765625f * (acc[r][5] - accz[5]);
#pragma unroll
        for (int v = 0; v < 4; ++v) res[r][v] = t[v] * 16777216.0f;
    }

    // lane (g, j) holds output rows i = 4g..4g+3 of weight row n0 + 16r + j
    if (NW == 1) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int i = 4 * g + v, n = n0 + 16 * r + j;
                if (i < M && n < N) Y[(int64_t)i * N + n] = __builtin_bit_cast(uint16_t, (_Float16)(res[r][v] * scale));
            }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[wv][r][4 * lane + v] = res[r][v];
        __syncthreads();
        for (int idx = threadIdx.x; idx < R * 256; idx += 64 * NW) {
            const int r = idx >> 8, l = (idx >> 2) & 63, v = idx & 3;
            const int i = 4 * (l >> 4) + v, n = n0 + 16 * r + (l & 15);
            if (i < M && n < N) {
                float s = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) s += red[w][r][idx & 255];
                Y[(int64_t)i * N + n] = __builtin_bit_cast(uint16_t, (_Float16)(s * scale));
            }
        }
    }
}

template <int FMT, int R, int NW>
static void launch_cfg(const uint16_t *X, const uint8_t *Wp, float scale, int M, int N, int K, int C, uint16_t *Y,
                       hipStream_t s)
{
    const int blocks = (N + 16 * R - 1) / (16 * R);
    hipLaunchKernelGGL((k_smallm<FMT, R, NW>), dim3(blocks), dim3(64 * NW), 0, s, X, Wp, scale, M, N, K, C, Y);
}

template <int FMT>
static void launch_fmt(const uint16_t *X, const uint8_t *Wp, float scale, int M, int N, int K, int C, uint16_t *Y,
                       hipStream_t s)
{
    // K split across up to 8 waves; two 16-row blocks per wave once M is large enough to
    // make the activation re-reads the larger cost
    if (C >= 64) {
        if (M > 8 && K <= 4096) launch_cfg<FMT, 2, 8>(X, Wp, scale, M, N, K, C, Y, s);
        else if (K <= 4096) launch_cfg<FMT, 1, 4>(X, Wp, scale, M, N, K, C, Y, s);
        else launch_cfg<FMT, 1, 8>(X, Wp, scale, M, N, K, C, Y, s);
    } else if (C >= 32) {
        launch_cfg<FMT, 1, 4>(X, Wp, scale, M, N, K, C, Y, s);
    } else if (C >= 16) {
        launch_cfg<FMT, 1, 2>(X, Wp, scale, M, N, K, C, Y, s);
    } else {
        launch_cfg<FMT, 1, 1>(X, Wp, scale, M, N, K, C, Y, s);
    }
}

int launch_smallm(const uint16_t *X, const uint8_t *Wp, float scale, int M, int N, int K, int fmt, uint16_t *Y,
                  hipStream_t s)
{
    const int C = (int)(row_bytes(K, fmt) / 16);
    if (fmt == TRI_FMT_2BIT) launch_fmt<TRI_FMT_2BIT>(X, Wp, scale, M, N, K, C, Y, s);
    else launch_fmt<TRI_FMT_1P6BIT>(X, Wp, scale, M, N, K, C, Y, s);
    return hipGetLastError() == hipSuccess ? TRI_OK : TRI_EHIP;
}

}  // namespace tri
