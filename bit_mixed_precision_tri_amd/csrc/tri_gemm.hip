// tri_gemm.hip -- ternary linear layer for many activation rows (prefill) on MFMA.
//
// The layer (Pith review of "Spectra 1.1", "What carries the argument"):
//   Y[m][n] = scale * sum_k t[n][k] * X[m][k],  t in {-1, 0, +1},  fp32 accumulation.
// Here it is a dense contraction (the review's "high-batch" regime), so it runs as a tiled
// fp16 MFMA GEMM (v_mfma_f32_32x32x16_f16) whose B operand is decoded from the packed
// trits in registers -- the gfx950 counterpart of the pages' FP16 x INT2 tensor-core
// kernel with fused dequantisation.
//
// Tiling.  A workgroup of 4 waves computes a 128 x 512 tile of Y; wave w owns output
// columns 128w..128w+127 (four 32-column MFMA tiles) for all 128 rows (four 32-row tiles):
// sixteen 32x32 accumulators, 256 accumulation registers.  Every A operand read from LDS
// feeds four MFMAs and every decoded B operand four.  K advances in tiles of one 32-byte
// packed slice per weight row: 128 trits (2-bit, 8 MFMA k-steps of 16) or 160 trits (1.6-bit,
// 10 k-steps).
//  - B (weights): lane (h = lane/32, c = lane%32) of column tile nt loads bytes 16h..16h+15
//    of the slice of weight row 32nt + c with one 16-byte buffer load (prefetched one K tile
//    ahead) and turns them into exact fp16 values of t: a 2-bit digit pair of a register,
//    moved to bits 0-1 / 16-17, is OR-ed into 1024.0 (0x6400) and 1025 is subtracted with one
//    packed fp16 add.  1.6-bit bytes first go through a 256-entry LDS table to the 2-bit
//    digit layout (five base-3 digits; the repeated division b'_i -> x_i that the review's
//    referee report describes for the paper's section 3.2), two bytes per register.
//  - Order of k: a 2-bit register pairs trits (16q+p, 16q+8+p) of its 16 and a 1.6-bit code
//    register trits (5r+p, 5r+20+p) of a 40-trit group; the sum over k is order-free, so the
//    activations are permuted the same way (v_perm_b32) when they are staged and no weight
//    byte is ever reshuffled.
//  - A (activations): each K tile of the 128 rows is loaded with buffer loads (rows past M
//    and values past K read as zero), permuted, and written to one of two LDS buffers in
//    k-step order ([k-step][h][8 values] per row), so an A operand is one 16-byte LDS read.
//  - Software pipeline: the 16 MFMAs of a k-step run while the A and B operands of the next
//    k-step are read and decoded; the next K tile is loaded at the start of a tile and
//    staged before its last k-step, where the single barrier of the tile sits.
// Workgroups are mapped to tiles XCD by XCD: consecutive workgroups of one XCD take
// consecutive row tiles of the same column tiles, so they share weights and activations in
// that XCD's L2.
#include <type_traits>

#include "tri_device.h"
#include "tri_internal.h"

namespace tri {

namespace {

constexpr uint32_t kRsrc3 = 0x00020000u;   // raw buffer resource, gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, (int)kRsrc3);
}

typedef float float16_t __attribute__((ext_vector_type(16)));

// v_mfma_f32_32x32x16_f16: D[32x32] += A[32x16] * B[16x32].  Lane (h = lane/32, l = lane%32)
// supplies A[l][k] and B[k][l] for the same eight k of half h, so any consistent order of k
// within an operand is a valid contraction; D[8i + 4h + v][l] is element 4i + v of the lane.
__device__ __forceinline__ float16_t mfma32(const u32x4 a, const u32x4 b, float16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c, 0,
                                                  0, 0);
}

// Exact fp16 pair (t_lo, t_hi) from the two 2-bit digits of `w` at bits 0-1 and 16-17:
// (w & 0x00030003) | 0x64006400 is (1024 + d_lo, 1024 + d_hi), and adding (-1025, -1025)
// leaves t = d - 1.  `bias` holds 0x64006400 in a vector register, so mask and bias fuse
// into one v_and_or_b32 (a gfx9 VOP3 instruction takes no literal and one scalar operand).
__device__ __forceinline__ uint32_t digits_to_t(uint32_t w, uint32_t bias)
{
    const uint32_t biased = (w & 0x00030003u) | bias;
    const half2_t r = as_h2(biased) + as_h2(0xE401E401u);
    return __builtin_bit_cast(uint32_t, r);
}

}  // namespace

constexpr int kBM = 128;             // rows of Y per workgroup
constexpr int kNT = 4;               // 32-column MFMA tiles per wave
constexpr int kMT = 4;               // 32-row MFMA tiles per wave
constexpr int kBN = 4 * 32 * kNT;    // columns of Y per workgroup (4 waves side by side)

template <int FMT>
__global__ __launch_bounds__(256) void k_gemm(const uint16_t *__restrict__ X, const uint8_t *__restrict__ Wp,
                                              float scale, int M, int N, int K, int C, int tiles_m, int tiles_n,
                                              uint16_t *__restrict__ Y)
{
    constexpr bool TWO = FMT == TRI_FMT_2BIT;
    constexpr int BK = TWO ? 128 : 160;          // trits per K tile (32 packed bytes per weight row)
    constexpr int KS = BK / 16;                  // MFMA k-steps per K tile
    constexpr int ASTR = BK + 8;                 // LDS row stride in halves (16 bytes of padding)
    constexpr int XP = BK / 8 / 2;               // 16-byte activation pieces per thread per K tile
    __shared__ uint16_t abuf[2][kBM * ASTR];
    __shared__ uint32_t lut[TWO ? 1 : 256];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps buffer descriptors scalar
    const int h = lane >> 5;
    const int c = lane & 31;

    // XCD-aware tile order: workgroups are dealt round-robin over 8 XCDs; renumber so that
    // the workgroups of one XCD are consecutive, then walk row tiles fastest.
    const int nwg = tiles_m * tiles_n;
    int bid = blockIdx.x;
    if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);
    const int tm = bid % tiles_m;
    const int tn = bid / tiles_m;
    const int m0 = tm * kBM;
    const int n0 = tn * kBN + 32 * kNT * wv;     // this wave's first column

    if constexpr (!TWO) {
        lut[tid] = base3_digits_2bit((uint32_t)tid);   // 256 threads, one entry each
    }

    // activations: thread -> (row tid/2, half ah = tid%2 of the K tile), XP 16-byte pieces
    const int arow = tid >> 1;
    const int ah = tid & 1;
    const uint32_t xbytes = __builtin_amdgcn_readfirstlane((uint32_t)((int64_t)min(kBM, M - m0) * K * 2));
    const __amdgpu_buffer_rsrc_t xr = rsrc(X + (int64_t)m0 * K, xbytes);
    // weights: lane (h, c) of column tile nt reads row n0 + 32nt + c, bytes 16h.. of each slice
    const int64_t S = (int64_t)C * 16;
    const int rows_here = min(32 * kNT, N - n0); // may be <= 0 for the last workgroup's high waves
    // (readfirstlane keeps the descriptor fields in scalar registers: a descriptor the compiler
    // believes divergent turns every buffer load into a loop)
    const uint32_t wbytes = __builtin_amdgcn_readfirstlane((uint32_t)((rows_here > 0 ? rows_here : 0) * S));
    const int wrow = __builtin_amdgcn_readfirstlane(min(n0, N - 1));
    const __amdgpu_buffer_rsrc_t wr = rsrc(Wp + (int64_t)wrow * S, wbytes);
    const int KT = (C + 1) / 2;                  // K tiles (two 16-byte chunks each)

    auto load_a = [&](int kt, u32x4 (&xa)[XP]) {
#pragma unroll
        for (int q = 0; q < XP; ++q) {
            const int k = kt * BK + ah * (BK / 2) + 8 * q;
            const uint32_t off = (uint32_t)(arow * K + k) * 2u;
            xa[q] = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)(k < K ? off : 0x80000000u), 0, 0);
        }
    };
    auto load_b = [&](int kt, u32x4 (&wb)[kNT]) {
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            const uint32_t off = (uint32_t)((32 * nt + c) * S + kt * 32 + 16 * h);
            wb[nt] = __builtin_amdgcn_raw_buffer_load_b128(wr, (int)off, 0, 0);
        }
    };
    // Permute this thread's half row of activations into the pairing of the decoded weights
    // and store it in k-step order: the values of k-step s for lane half ah sit at 16s + 8ah.
    auto store_a = [&](int buf, const u32x4 (&xa)[XP]) {
        uint16_t *dst = &abuf[buf][arow * ASTR + 8 * ah];
        uint32_t v[XP * 4];
#pragma unroll
        for (int q = 0; q < XP; ++q) {
            v[4 * q] = xa[q][0]; v[4 * q + 1] = xa[q][1]; v[4 * q + 2] = xa[q][2]; v[4 * q + 3] = xa[q][3];
        }
        uint32_t o[XP * 4];
        if constexpr (TWO) {
            // each 16-value group q: (x0,x8),(x1,x9),...,(x7,x15); k-steps 2q and 2q+1
#pragma unroll
            for (int w = 0; w < XP * 4 / 8; ++w)
#pragma unroll
                for (int p = 0; p < 8; p += 2) {
                    o[8 * w + p] = pair_halves<0>(v[8 * w + 4 + p / 2], v[8 * w + p / 2]);
                    o[8 * w + p + 1] = pair_halves<1>(v[8 * w + 4 + p / 2], v[8 * w + p / 2]);
                }
        } else {
            // each 40-value group gg: for p = 0..4, r = 0..3: (x[5r+p], x[5r+20+p]); k-steps 5gg+p
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
        for (int s = 0; s < KS; ++s)
            *reinterpret_cast<u32x4 *>(dst + 16 * s) = u32x4{o[4 * s], o[4 * s + 1], o[4 * s + 2], o[4 * s + 3]};
    };

    float16_t acc[kMT][kNT];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) acc[mt][nt] = float16_t{};
    uint32_t bias;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(bias));   // register-held constant (no memory access)

    // Weight source registers of the current K tile: the packed dwords (2-bit) or the digit
    // codes of byte pairs (b, b + 4) of each 8-byte half (1.6-bit).
    constexpr int SW = TWO ? 4 : 8;
    uint32_t src[kNT][SW];
    u32x4 xa[XP];
    u32x4 wn[kNT];
    auto take_b = [&]() {
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            if constexpr (TWO) {
#pragma unroll
                for (int q = 0; q < 4; ++q) src[nt][q] = wn[nt][q];
            } else {
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) {
                    const uint32_t lo = wn[nt][2 * (cc >> 2)], hi = wn[nt][2 * (cc >> 2) + 1];
                    const int sh = 8 * (cc & 3);
                    src[nt][cc] = lut[(lo >> sh) & 0xFFu] | (lut[(hi >> sh) & 0xFFu] << 16);
                }
            }
        }
    };
    // B operand of k-step s, column tile nt
    auto decode = [&](int s, int nt) {
        u32x4 b;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if constexpr (TWO)
                b[r] = digits_to_t(src[nt][s >> 1] >> (2 * (4 * (s & 1) + r)), bias);
            else
                b[r] = digits_to_t(src[nt][4 * (s / 5) + r] >> (2 * (s % 5)), bias);
        }
        return b;
    };

    load_a(0, xa);
    load_b(0, wn);
    store_a(0, xa);
    __syncthreads();                             // tile 0's activations and the byte table
    take_b();
    const int aoff = c * ASTR + 8 * h;
    u32x4 afr[kMT], bop[kNT];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) afr[mt] = *reinterpret_cast<const u32x4 *>(&abuf[0][aoff + 32 * mt * ASTR]);
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) bop[nt] = decode(0, nt);

    // One K tile; MORE (a compile-time flag, so the tile body has no branches) says whether a
    // next tile exists.
    auto tile = [&](int kt, auto more_tag) {
        constexpr bool MORE = decltype(more_tag)::value;
        const int buf = kt & 1;
        if constexpr (MORE) {
            load_a(kt + 1, xa);
            load_b(kt + 1, wn);
        }
        const uint16_t *acur = &abuf[buf][aoff];
        const uint16_t *anext = &abuf[buf ^ 1][aoff];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            // every wave has stored its share of the next tile (step KS - 2) and read its
            // last operands of this one: the next tile's buffer may be read from here on
            if (MORE && s == KS - 1) __syncthreads();
            u32x4 an[kMT], bn[kNT];
            if (s + 1 < KS) {
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt)
                    an[mt] = *reinterpret_cast<const u32x4 *>(acur + 32 * mt * ASTR + 16 * (s + 1));
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) bn[nt] = decode(s + 1, nt);
            } else if (MORE) {
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt) an[mt] = *reinterpret_cast<const u32x4 *>(anext + 32 * mt * ASTR);
                take_b();                        // the last decode of this tile's words was at step KS - 2
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) bn[nt] = decode(0, nt);
            }
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) acc[mt][nt] = mfma32(afr[mt], bop[nt], acc[mt][nt]);
            if (MORE && s == KS - 2) store_a(buf ^ 1, xa);
            // interleave: each MFMA is followed by a share of the next step's decode and reads
#pragma unroll
            for (int i = 0; i < kMT * kNT; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // 3 VALU
                if (i % 4 == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
            }
            __builtin_amdgcn_sched_barrier(0);
            if (s + 1 < KS || MORE) {
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt) afr[mt] = an[mt];
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) bop[nt] = bn[nt];
            }
        }
    };
    for (int kt = 0; kt + 1 < KT; ++kt) tile(kt, std::true_type{});
    tile(KT - 1, std::false_type{});

    // epilogue: lane (h, c) holds rows 32mt + 8i + 4h + v of column 32nt + c
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            const int n = n0 + 32 * nt + c;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int m = m0 + 32 * mt + 8 * i + 4 * h + v;
                    if (m < M && n < N)
                        Y[(int64_t)m * N + n] = __builtin_bit_cast(uint16_t, (_Float16)(acc[mt][nt][4 * i + v] * scale));
                }
        }
}

int launch_gemm(const uint16_t *X, const uint8_t *Wp, float scale, int64_t M, int N, int K, int fmt, uint16_t *Y,
                hipStream_t s)
{
    const int C = (int)(row_bytes(K, fmt) / 16);
    const int64_t S = (int64_t)C * 16;
    // 32-bit buffer offsets: a 128-row activation block and a 128-row weight block must stay
    // below 2^31 bytes, and activations are read in pieces of 8 values (K % 8 == 0).  Other
    // shapes run the small-M kernels over 16-row slices of X.
    const bool fits = (K % 8) == 0 && (int64_t)kBM * K * 2 < ((int64_t)1 << 31) && 32 * kNT * S < ((int64_t)1 << 31);
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
