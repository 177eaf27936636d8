// tri_gemm.hip -- ternary linear layer for many activation rows (prefill) on MFMA.
//
// The layer (Pith review of "Spectra 1.1", "What carries the argument"):
//   Y[m][n] = scale * sum_k t[n][k] * X[m][k],  t in {-1, 0, +1},  fp32 accumulation.
// Here it is a dense contraction (the review's "high-batch" regime), so it runs as a tiled
// fp16 MFMA GEMM (v_mfma_f32_16x16x32_f16) whose B operand is decoded from the packed
// trits in registers -- the gfx950 counterpart of the pages' FP16 x INT2 tensor-core
// kernel with fused dequantisation.
//
// Tiling.  A workgroup of 4 waves computes a 128 x 256 tile of Y; wave w owns output
// columns 64w..64w+63 (four 16-column MFMA tiles) for all 128 rows (eight 16-row tiles), so
// no two waves decode the same weights.  K advances in tiles of one 32-byte packed slice
// per weight row: 128 trits (2-bit) or 160 trits (1.6-bit).
//  - A (activations): each K tile of the 128 rows is loaded with buffer loads (rows past M
//    and values past K read as zero), permuted in place into the pairing of the decoded
//    weights, and written to one of two LDS buffers while the MFMAs of the previous tile
//    run; one barrier per K tile.
//  - B (weights): lane (g = lane/16, j = lane%16) loads the 8 packed bytes 8g..8g+7 of the
//    slice of weight row 16*nt + j straight into registers (prefetched one K tile ahead)
//    and turns them into exact fp16 values of t: the 2-bit digit pair of a register, moved
//    to bits 0-1 / 16-17, is OR-ed into 1024.0 (0x6400) and 1025 is subtracted with one
//    packed fp16 add.  1.6-bit bytes first go through a 256-entry LDS table to the 2-bit
//    digit layout (five base-3 digits; the repeated division b'_i -> x_i that the review's
//    referee report describes for the paper's section 3.2).
//  - Order of k: a 2-bit register pairs trits (16w+p, 16w+8+p) and a 1.6-bit one trits
//    (5r+p, 5r+20+p) of an 8-byte group; the sum over k is order-free, so the activations
//    are permuted the same way (v_perm_b32) and no weight byte is ever reshuffled.
// Workgroups are mapped to tiles XCD by XCD: consecutive workgroups of one XCD take
// consecutive row tiles of the same column tiles, so they share weights and activations in
// that XCD's L2.
#include "tri_device.h"
#include "tri_internal.h"

namespace tri {

namespace {

constexpr uint32_t kRsrc3 = 0x00020000u;   // raw buffer resource, gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, (int)kRsrc3);
}

__device__ __forceinline__ float4_t mfma_t(const u32x4 a, const u32x4 b, float4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c, 0,
                                                  0, 0);
}

// Exact fp16 pair (t_lo, t_hi) from two 2-bit digits sitting at bits 0-1 and 16-17.
__device__ __forceinline__ uint32_t digits_to_t(uint32_t d01)
{
    const uint32_t biased = d01 | 0x64006400u;                  // (1024 + d_lo, 1024 + d_hi)
    const half2_t r = as_h2(biased) + as_h2(0xE401E401u);        // + (-1025, -1025)
    return __builtin_bit_cast(uint32_t, r);
}

}  // namespace

constexpr int kBM = 128;     // rows of Y per workgroup
constexpr int kBN = 256;     // columns of Y per workgroup

template <int FMT>
__global__ __launch_bounds__(256) void k_gemm(const uint16_t *__restrict__ X, const uint8_t *__restrict__ Wp,
                                              float scale, int M, int N, int K, int C, int tiles_m, int tiles_n,
                                              uint16_t *__restrict__ Y)
{
    constexpr bool TWO = FMT == TRI_FMT_2BIT;
    constexpr int BK = TWO ? 128 : 160;          // trits per K tile (32 packed bytes per weight row)
    constexpr int KS = BK / 32;                  // MFMA k-steps per K tile
    constexpr int GH = BK / 4;                   // activations per lane group and K tile
    constexpr int ASTR = BK + 8;                 // LDS row stride in halves (16 bytes of padding)
    constexpr int XP = BK / 8 / 2;               // 16-byte activation pieces per thread per K tile
    __shared__ uint16_t abuf[2][kBM * ASTR];
    __shared__ uint32_t lut[TWO ? 1 : 256];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int g = lane >> 4;
    const int j = lane & 15;

    // XCD-aware tile order: workgroups are dealt round-robin over 8 XCDs; renumber so that
    // the workgroups of one XCD are consecutive, then walk row tiles fastest.
    const int nwg = tiles_m * tiles_n;
    int bid = blockIdx.x;
    if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);
    const int tm = bid % tiles_m;
    const int tn = bid / tiles_m;
    const int m0 = tm * kBM;
    const int n0 = tn * kBN + 64 * wv;           // this wave's first column

    if constexpr (!TWO) {
        lut[tid] = base3_digits_2bit((uint32_t)tid);   // 256 threads, one entry each
    }

    // activations: thread -> (row tid/2, half tid%2 of the K tile), XP 16-byte pieces
    const int arow = tid >> 1;
    const int acol0 = (tid & 1) * (BK / 2);
    const __amdgpu_buffer_rsrc_t xr = rsrc(X + (int64_t)m0 * K, (uint32_t)((int64_t)min(kBM, M - m0) * K * 2));
    // weights: lane (g, j) of column tile nt reads row n0 + 16nt + j, bytes 8g.. of each slice
    const int64_t S = (int64_t)C * 16;
    const int rows_here = min(64, N - n0);       // may be <= 0 for the last workgroup's high waves
    const __amdgpu_buffer_rsrc_t wr =
        rsrc(Wp + (int64_t)min(n0, N - 1) * S, (uint32_t)((rows_here > 0 ? rows_here : 0) * S));
    const int KT = (C + 1) / 2;                  // K tiles (two 16-byte chunks each)

    auto load_a = [&](int kt, u32x4 (&xa)[XP]) {
#pragma unroll
        for (int q = 0; q < XP; ++q) {
            const int k = kt * BK + acol0 + 8 * q;
            const uint32_t off = (uint32_t)(arow * K + k) * 2u;
            xa[q] = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)(k < K ? off : 0x80000000u), 0, 0);
        }
    };
    auto load_b = [&](int kt, uint32_t (&wb)[4][2]) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const uint32_t off = (uint32_t)((16 * nt + j) * S + kt * 32 + 8 * g);
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(wr, (int)off, 0, 0);
            wb[nt][0] = v[0];
            wb[nt][1] = v[1];
        }
    };
    // permute the activations in place (the pairing of the decoded weights) and store to LDS
    auto store_a = [&](int buf, const u32x4 (&xa)[XP]) {
        uint16_t *dst = &abuf[buf][arow * ASTR + acol0];
        uint32_t v[XP * 4];
#pragma unroll
        for (int q = 0; q < XP; ++q) {
            v[4 * q] = xa[q][0]; v[4 * q + 1] = xa[q][1]; v[4 * q + 2] = xa[q][2]; v[4 * q + 3] = xa[q][3];
        }
        uint32_t o[XP * 4];
        if constexpr (TWO) {
            // each 16-value group: (x0,x8),(x1,x9),...,(x7,x15)
#pragma unroll
            for (int w = 0; w < XP * 4 / 8; ++w)
#pragma unroll
                for (int p = 0; p < 8; p += 2) {
                    o[8 * w + p] = pair_halves<0>(v[8 * w + 4 + p / 2], v[8 * w + p / 2]);
                    o[8 * w + p + 1] = pair_halves<1>(v[8 * w + 4 + p / 2], v[8 * w + p / 2]);
                }
        } else {
            // each 40-value group: for p = 0..4, r = 0..3: (x[5r+p], x[5r+20+p])
#pragma unroll
            for (int gg = 0; gg < XP * 4 / 20; ++gg)
#pragma unroll
                for (int p = 0; p < 5; ++p)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int e = 5 * r + p;           // value index in the group; partner e + 20
                        o[20 * gg + 4 * p + r] = (e & 1) ? pair_halves<1>(v[20 * gg + (e >> 1) + 10], v[20 * gg + (e >> 1)])
                                                         : pair_halves<0>(v[20 * gg + (e >> 1) + 10], v[20 * gg + (e >> 1)]);
                    }
        }
#pragma unroll
        for (int q = 0; q < XP; ++q)
            reinterpret_cast<u32x4 *>(dst)[q] = u32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
    };

    const float4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    float4_t acc[8][4];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = zero4;

    u32x4 xa[XP];
    uint32_t wb[4][2];
    load_a(0, xa);
    load_b(0, wb);
    store_a(0, xa);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        uint32_t wn[4][2];
        if (kt + 1 < KT) {                       // prefetch the next K tile
            load_a(kt + 1, xa);
            load_b(kt + 1, wn);
        }
        // B operands of this K tile: per column tile, KS operands of 4 registers
        u32x4 bop[4][KS];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            if constexpr (TWO) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const uint32_t w = wb[nt][ks >> 1];
                    const int p0 = 4 * (ks & 1);
                    u32x4 b;
#pragma unroll
                    for (int r = 0; r < 4; ++r) b[r] = digits_to_t((w >> (2 * (p0 + r))) & 0x00030003u);
                    bop[nt][ks] = b;
                }
            } else {
                uint32_t code[4];                // bytes r and r+4 of the 8-byte group, as digit codes
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    code[r] = lut[(wb[nt][0] >> (8 * r)) & 0xFFu] | (lut[(wb[nt][1] >> (8 * r)) & 0xFFu] << 16);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    u32x4 b;
#pragma unroll
                    for (int r = 0; r < 4; ++r) b[r] = digits_to_t((code[r] >> (2 * ks)) & 0x00030003u);
                    bop[nt][ks] = b;
                }
            }
        }
        // MFMAs: A from LDS (lane (g, i): row 16mt + i, activations GH*g + 8ks ..)
        const uint16_t *abase = &abuf[buf][j * ASTR + GH * g];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(abase + 16 * mt * ASTR + 8 * ks);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma_t(a, bop[nt][ks], acc[mt][nt]);
            }
        }
        if (kt + 1 < KT) {
            store_a(buf ^ 1, xa);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                wb[nt][0] = wn[nt][0];
                wb[nt][1] = wn[nt][1];
            }
        }
        __syncthreads();
    }

    // epilogue: lane (g, j) holds rows 16mt + 4g + v of column 16nt + j
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int n = n0 + 16 * nt + j;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + 16 * mt + 4 * g + v;
                if (m < M && n < N)
                    Y[(int64_t)m * N + n] = __builtin_bit_cast(uint16_t, (_Float16)(acc[mt][nt][v] * scale));
            }
        }
}

int launch_gemm(const uint16_t *X, const uint8_t *Wp, float scale, int64_t M, int N, int K, int fmt, uint16_t *Y,
                hipStream_t s)
{
    const int C = (int)(row_bytes(K, fmt) / 16);
    const int64_t S = (int64_t)C * 16;
    // 32-bit buffer offsets: a 128-row activation block and a 64-row weight block must stay
    // below 2^31 bytes, and activations are read in pieces of 8 values (K % 8 == 0).  Other
    // shapes run the small-M kernels over 16-row slices of X.
    const bool fits = (K % 8) == 0 && (int64_t)kBM * K * 2 < ((int64_t)1 << 31) && 64 * S < ((int64_t)1 << 31);
    if (!fits) {
        for (int64_t m0 = 0; m0 < M; m0 += 16) {
            const int mm = (int)((M - m0) < 16 ? (M - m0) : 16);
            const int rc = launch_smallm(X + m0 * K, Wp, scale, mm, N, K, fmt, Y + m0 * N, s);
            if (rc != TRI_OK) return rc;
        }
        return TRI_OK;
    }
    for (int64_t mb = 0; mb < M; mb += (int64_t)1 << 24) {   // grid.x limit: 2^24 row tiles per launch
        const int mm = (int)((M - mb) < ((int64_t)1 << 24) ? (M - mb) : ((int64_t)1 << 24));
        const int tiles_m = (mm + kBM - 1) / kBM;
        const int tiles_n = (N + kBN - 1) / kBN;
        const int64_t nwg = (int64_t)tiles_m * tiles_n;
        if (nwg >= ((int64_t)1 << 31)) return TRI_EINVAL;
        if (fmt == TRI_FMT_2BIT)
            hipLaunchKernelGGL(k_gemm<TRI_FMT_2BIT>, dim3((unsigned)nwg), dim3(256), 0, s, X + mb * K, Wp, scale, mm,
                               N, K, C, tiles_m, tiles_n, Y + mb * N);
        else
            hipLaunchKernelGGL(k_gemm<TRI_FMT_1P6BIT>, dim3((unsigned)nwg), dim3(256), 0, s, X + mb * K, Wp, scale,
                               mm, N, K, C, tiles_m, tiles_n, Y + mb * N);
        if (hipGetLastError() != hipSuccess) return TRI_EHIP;
    }
    return TRI_OK;
}

}  // namespace tri
