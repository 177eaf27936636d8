// tri_mvm.hip -- ternary linear layer for a few activation rows (2 <= M <= 16, batched decode)
// on MFMA.
//
// The layer (Pith review of "Spectra 1.1", "What carries the argument"):
//   Y[m][n] = scale * sum_k t[n][k] * X[m][k],  t in {-1, 0, +1},  fp32 accumulation.
// v_mfma_f32_16x16x32_f16 takes the (up to) 16 activation rows as its A operand and 16 weight
// rows, decoded in registers, as B.  The decode is the one of the M = 1 kernel (tri_mv1.hip):
// masked digits d = t + 1 read as exact fp16 values d * 4^p * 2^-24, one MFMA and one
// accumulator per position class, classes merged with exact powers of two, and
// sum_k X[m][k] subtracted once per output at the end.
//
// Work split.  A workgroup of NW waves owns 16 weight rows; wave w takes chunk-steps s, where
// lane (g = lane/16, j = lane%16) reads 16-byte chunk c = 4*(s*NW + w) + g of weight row j and
// supplies the activations of row j of X (as A operand) for the same chunk.  All weight chunks
// of the wave are requested at the start.  The activations of a step -- four consecutive
// chunks of every activation row -- are read with whole-line loads one step ahead, bounced
// through the wave's LDS slot to the lanes that use them, and permuted there into the
// pairing of the decoded weights (2-bit: trits (16v+p, 16v+8+p); 1.6-bit: (5q+p, 5q+40+p)).
// The waves' partial tiles are added in LDS in a fixed order (no atomics).
#include "tri_device.h"
#include "tri_internal.h"

namespace tri {

namespace {

constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer resource, gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

__device__ __forceinline__ float4_t mfma(const u32x4 a, const u32x4 b, float4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c, 0,
                                                  0, 0);
}

__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace

template <int FMT, int MT, int NW, int CST>
__global__ __launch_bounds__(64 * NW) void k_mvm(const uint16_t *__restrict__ X, const Groups gr, int M, int K, int C)
{
    const int gi = group_of(gr, (int)blockIdx.x);
    const uint8_t *__restrict__ Wp = gr.Wp[gi];
    uint16_t *__restrict__ Y = gr.Y[gi];
    const float scale = gr.scale[gi];
    const int N = gr.N[gi];
    constexpr bool TWO = FMT == TRI_FMT_2BIT;
    constexpr int XH = TWO ? 64 : 80;            // activations per chunk
    constexpr int NOP = TWO ? 8 : 10;            // A operands (MFMAs) per chunk
    constexpr int NCLS = TWO ? 6 : 5;            // position classes
    constexpr int RP = 4 * XH / 8;               // 16-byte pieces of one row per step (32 or 40)
    constexpr int NLD = (MT * RP + 63) / 64;     // whole-line activation loads per lane and step
    constexpr int RPP = RP + 1;                  // padded row stride: the 16 rows a read touches fall in distinct banks
    __shared__ u32x4 xraw[NW][MT * RPP];         // per wave: one step's activations, row-major
    __shared__ uint32_t lut[TWO ? 1 : 256];
    __shared__ float red[NW][16][17];            // per wave: partial tile [row m][column j], + sum x

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (scalar descriptors)
    const int g = lane >> 4;
    const int j = lane & 15;
    const int n0 = ((int)blockIdx.x - gr.blk[gi]) * 16;
    const int64_t S = (int64_t)C * 16;

    if constexpr (!TWO) {
        for (int b = threadIdx.x; b < 256; b += 64 * NW) lut[b] = base3_digits_2bit((uint32_t)b);
        __syncthreads();
    }

    // every weight chunk of the wave, all in flight at once
    const int rows_here = min(16, N - n0);
    const __amdgpu_buffer_rsrc_t wr =
        rsrc(Wp + (int64_t)n0 * S, __builtin_amdgcn_readfirstlane((uint32_t)(rows_here * S)));
    u32x4 wq[CST];
#pragma unroll
    for (int s = 0; s < CST; ++s) {
        const int c = 4 * (s * NW + wv) + g;
        wq[s] = __builtin_amdgcn_raw_buffer_load_b128(wr, (int)(c < C ? (uint32_t)(j * S + c * 16) : 0x80000000u), 0, 0);
    }
    // activations of step s: piece P = 64i + lane is piece P % RP of row P / RP, i.e. values
    // 16*(4*(s*NW + w)*XH/16 + P % RP) ... of that row: whole 128-byte lines per instruction
    const __amdgpu_buffer_rsrc_t xr = rsrc(X, __builtin_amdgcn_readfirstlane((uint32_t)((int64_t)M * K * 2)));
    auto load_x = [&](int s, u32x4 (&xv)[NLD]) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int P = 64 * i + lane;
            const int row = P / RP;
            const int k = 4 * (s * NW + wv) * XH + 8 * (P % RP);
            const bool live = row < M && k < K;
            xv[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)(live ? (uint32_t)(row * K + k) * 2u : 0x80000000u),
                                                          0, 0);
        }
    };

    const float4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    float4_t acc[NCLS];
#pragma unroll
    for (int c = 0; c < NCLS; ++c) acc[c] = zero4;
    float4_t accx = zero4;                       // sum_k X[m][k] in every column of the tile
    // the activations of PD steps are in flight at once (a ring of register sets; one step
    // ahead measured best: deeper rings gained nothing)
    constexpr int PD = 1;
    u32x4 xv[PD][NLD];
#pragma unroll
    for (int t = 0; t < PD; ++t) load_x(t, xv[t]);
#pragma unroll
    for (int s = 0; s < CST; ++s) {
        if (4 * (s * NW + wv) >= C) break;       // wave-uniform: no chunk of this step is live
        // bounce the step's raw activations to the lanes that use them, then permute there
#pragma unroll
        for (int i = 0; i < NLD; ++i)
            if (64 * i + lane < MT * RP) xraw[wv][64 * i + lane + (64 * i + lane) / RP] = xv[s % PD][i];
        wave_sync();
        if (s + PD < CST) load_x(s + PD, xv[s % PD]);   // refill the set just emptied
        uint32_t x32[XH / 2];                    // row j, chunk g of the step (zero past the tile's rows)
#pragma unroll
        for (int q = 0; q < XH / 8; ++q) {
            const u32x4 v = j < MT ? xraw[wv][j * RPP + (XH / 8) * g + q] : u32x4{0u, 0u, 0u, 0u};
            x32[4 * q] = v[0]; x32[4 * q + 1] = v[1]; x32[4 * q + 2] = v[2]; x32[4 * q + 3] = v[3];
        }
        wave_sync();                             // the slot may be refilled at the next step
        u32x4 a[NOP];
        if constexpr (TWO) {
#pragma unroll
            for (int p = 0; p < 8; ++p)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    a[p][v] = (p & 1) ? pair_halves<1>(x32[8 * v + 4 + p / 2], x32[8 * v + p / 2])
                                      : pair_halves<0>(x32[8 * v + 4 + p / 2], x32[8 * v + p / 2]);
        } else {
#pragma unroll
            for (int p = 0; p < 5; ++p)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq) {
                        const int e = 5 * (4 * hh + qq) + p;   // value index; partner e + 40
                        a[2 * p + hh][qq] = (e & 1) ? pair_halves<1>(x32[(e >> 1) + 20], x32[e >> 1])
                                                    : pair_halves<0>(x32[(e >> 1) + 20], x32[e >> 1]);
                    }
        }
        // sum_k X[m][k] on the matrix cores: every A operand against a B of ones
        const u32x4 ones = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
#pragma unroll
        for (int p = 0; p < NOP; ++p) accx = mfma(a[p], ones, accx);
        // decode and contract
        const u32x4 v = wq[s];
        if constexpr (TWO) {
            const u32x4 u = v >> 12u;
#pragma unroll
            for (int p = 0; p < 6; ++p) acc[p] = mfma(a[p], v & (0x00030003u << (2 * p)), acc[p]);
            acc[0] = mfma(a[6], u & 0x00030003u, acc[0]);
            acc[1] = mfma(a[7], u & 0x000C000Cu, acc[1]);
        } else {
            u32x4 lo, hi;
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
                acc[p] = mfma(a[2 * p], lo & m, acc[p]);
                acc[p] = mfma(a[2 * p + 1], hi & m, acc[p]);
            }
        }
    }

    // merge classes: lane (g, j) holds rows 4g + e of column j (of D and of the sums of X)
    float4_t t = acc[0] + 0.25f * acc[1];
    t += 0.0625f * acc[2] + 0.015625f * acc[3];
    t += 0.00390625f * acc[4];
    if constexpr (TWO) t += 0.0009765625f * acc[5];
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wv][4 * g + e][j] = t[e];
    if (j == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wv][4 * g + e][16] = accx[e];
    }
    __syncthreads();
    // thread (m, jj): output Y[m][n0 + jj], waves added in a fixed order
    for (int o = threadIdx.x; o < MT * 16; o += 64 * NW) {
        const int m = o >> 4, jj = o & 15;
        if (m < M && n0 + jj < N) {
            float sd = 0.f, sx = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                sd += red[w][m][jj];
                sx += red[w][m][16];
            }
            Y[(int64_t)m * N + n0 + jj] = __builtin_bit_cast(uint16_t, (_Float16)((sd * 16777216.0f - sx) * scale));
        }
    }
}

template <int FMT, int MT, int NW, int CST>
static void launch_cfg(const uint16_t *X, const Groups &gr, int M, int K, int C, hipStream_t s)
{
    hipLaunchKernelGGL((k_mvm<FMT, MT, NW, CST>), dim3(gr.blk[gr.G]), dim3(64 * NW), 0, s, X, gr, M, K, C);
}

template <int FMT, int MT>
static bool launch_mt(const uint16_t *X, const Groups &gr, int M, int K, int C, hipStream_t s)
{
    const int cst8 = (C + 31) / 32;              // chunk-steps with 8 waves (4 chunks per step and wave)
    switch (cst8) {
    case 1: launch_cfg<FMT, MT, 8, 1>(X, gr, M, K, C, s); return true;
    case 2: launch_cfg<FMT, MT, 8, 2>(X, gr, M, K, C, s); return true;
    case 3: launch_cfg<FMT, MT, 8, 3>(X, gr, M, K, C, s); return true;
    case 4: launch_cfg<FMT, MT, 8, 4>(X, gr, M, K, C, s); return true;
    case 5: launch_cfg<FMT, MT, 8, 5>(X, gr, M, K, C, s); return true;
    case 6: launch_cfg<FMT, MT, 8, 6>(X, gr, M, K, C, s); return true;
    case 7: launch_cfg<FMT, MT, 8, 7>(X, gr, M, K, C, s); return true;
    case 8: launch_cfg<FMT, MT, 8, 8>(X, gr, M, K, C, s); return true;
    default: break;
    }
    // sixteen waves, while the per-wave activation slots fit in LDS
    if constexpr (FMT == TRI_FMT_2BIT || MT <= 8) {
        const int cst16 = (C + 63) / 64;
        if (cst16 <= 8) { launch_cfg<FMT, MT, 16, 8>(X, gr, M, K, C, s); return true; }
        if (cst16 <= 16) { launch_cfg<FMT, MT, 16, 16>(X, gr, M, K, C, s); return true; }
    }
    return false;                                // longer rows: the streaming small-M kernel
}

bool launch_mvm(const uint16_t *X, const Groups &gr, int M, int K, int fmt, hipStream_t s)
{
    const int C = (int)(row_bytes(K, fmt) / 16);
    // 32-bit buffer offsets: the activations and one 16-row block stay below 2^31 bytes;
    // activations are read in pieces of 8 values, so K must be a multiple of 8
    if (M < 2 || M > 16 || (K % 8) != 0 || (int64_t)M * K * 2 >= ((int64_t)1 << 31) ||
        16 * (int64_t)C * 16 >= ((int64_t)1 << 31))
        return false;
    const bool two = fmt == TRI_FMT_2BIT;
    if (M <= 4) return two ? launch_mt<TRI_FMT_2BIT, 4>(X, gr, M, K, C, s) : launch_mt<TRI_FMT_1P6BIT, 4>(X, gr, M, K, C, s);
    if (M <= 8) return two ? launch_mt<TRI_FMT_2BIT, 8>(X, gr, M, K, C, s) : launch_mt<TRI_FMT_1P6BIT, 8>(X, gr, M, K, C, s);
    return two ? launch_mt<TRI_FMT_2BIT, 16>(X, gr, M, K, C, s) : launch_mt<TRI_FMT_1P6BIT, 16>(X, gr, M, K, C, s);
}

}  // namespace tri
