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
constexpr int kBN = 512;             // columns of Y per tile (4 waves side by side, 4 MFMA tiles each)

// A workgroup computes one BM x 512 tile of Y (NT = 4), one half of it, BM x 256 (NT = 2), or one
// quarter, BM x 128 (NT = 1): part blockIdx.x % (4/NT) of tile tile_base + blockIdx.x / (4/NT) in
// the tile order.  BM is 128, or 64 for a middling M (each wave then covers 64 rows).
template <int FMT, int NT, int BM>
__global__ __launch_bounds__(256) void k_gemm(const uint16_t *__restrict__ X, const uint8_t *__restrict__ Wp,
                                              float scale, int M, int N, int K, int C, int tiles_m, int tiles_n,
                                              int tile_base, uint16_t *__restrict__ Y)
{
    constexpr int kNT = NT;                      // 32-column MFMA tiles per wave
    constexpr int kBMt = BM;                     // rows of Y per workgroup (128, or 64 for few rows)
    constexpr int kMTt = BM / 32;                // 32-row MFMA tiles per wave
    static_assert(BM == 128 || BM == 64, "tile heights");
    constexpr bool TWO = FMT == TRI_FMT_2BIT;
    constexpr int BK = TWO ? 128 : 160;          // trits per K tile (32 packed bytes per weight row)
    constexpr int KS = BK / 16;                  // MFMA k-steps per K tile
    constexpr int ASTR = BK + 8;                 // LDS row stride in halves (16 bytes of padding)
    // activation groups: the values whose weight trits share decode registers (16 for 2-bit,
    // 40 for 1.6-bit); a thread loads whole groups, lanes walking along a row
    constexpr int GV = TWO ? 16 : 40;            // values per group
    constexpr int GPR = BK / GV;                 // groups per row and K tile (8 or 4)
    constexpr int GP = GV / 8;                   // 16-byte pieces per group
    constexpr int NG = kBMt * GPR / 256;          // groups per thread and K tile
    constexpr int XP = NG * GP;                  // 16-byte pieces per thread and K tile
    __shared__ uint16_t abuf[2][kBMt * ASTR];
    __shared__ uint32_t lut[TWO ? 1 : 256];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps buffer descriptors scalar
    const int h = lane >> 5;
    const int c = lane & 31;

    // Tile order.  Workgroups are dealt round-robin over the 8 XCDs; renumber them so that
    // each XCD gets a contiguous range, and walk the tiles in bands of kGM row tiles: the 32
    // workgroups an XCD runs at once then cover 4 row tiles x 8 column tiles and share
    // activations and weights in that XCD's L2.
    constexpr int kGM = 4;
    const int nwg = gridDim.x;
    int bid = blockIdx.x;
    if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);
    constexpr int kParts = 4 / NT;               // workgroups per 128 x 512 tile
    static_assert(NT == 1 || NT == 2 || NT == 4, "tile widths");
    const int t = tile_base + bid / kParts;
    const int band = t / (kGM * tiles_n);
    const int first_m = band * kGM;
    const int band_m = min(tiles_m - first_m, kGM);
    const int in_band = t - band * kGM * tiles_n;
    const int tm = first_m + in_band % band_m;
    const int tn = in_band / band_m;
    const int m0 = tm * kBMt;
    const int n0 = tn * kBN + (bid % kParts) * (kBN / kParts) + 32 * kNT * wv;   // this wave's first column

    if constexpr (!TWO) {
        lut[tid] = base3_digits_2bit((uint32_t)tid);   // 256 threads, one entry each
    }

    const uint32_t xbytes = __builtin_amdgcn_readfirstlane((uint32_t)((int64_t)min(kBMt, M - m0) * K * 2));
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

    // Activations of K tile kt (tiles past the end read zeros: the k < K test and the
    // buffer range check); group gi = q*256 + tid is group gi % GPR of row gi / GPR.
    auto load_a = [&](int kt, u32x4 (&xa)[XP]) {
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            const int gi = q * 256 + tid;
            const int row = gi / GPR, G = gi % GPR;
#pragma unroll
            for (int j = 0; j < GP; ++j) {
                const int k = kt * BK + GV * G + 8 * j;
                const uint32_t off = (uint32_t)(row * K + k) * 2u;
                xa[q * GP + j] = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)(k < K ? off : 0x80000000u), 0, 0);
            }
        }
    };
    // Weights of K tile kt (a tile past the end reads bytes that are never used, within range).
    auto load_b = [&](int kt, u32x4 (&wb)[kNT]) {
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            const uint32_t off = (uint32_t)((32 * nt + c) * S + kt * 32 + 16 * h);
            wb[nt] = __builtin_amdgcn_raw_buffer_load_b128(wr, (int)off, 0, 0);
        }
    };
    // Permute each group into the pairing of the decoded weights and store it in k-step
    // order: the 8 values lane half hh uses at k-step s sit at 16s + 8hh of the row.
    auto store_a = [&](int buf, const u32x4 (&xa)[XP]) {
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            const int gi = q * 256 + tid;
            const int row = gi / GPR, G = gi % GPR;
            uint32_t v[GV / 2];
#pragma unroll
            for (int j = 0; j < GP; ++j) {
                v[4 * j] = xa[q * GP + j][0]; v[4 * j + 1] = xa[q * GP + j][1];
                v[4 * j + 2] = xa[q * GP + j][2]; v[4 * j + 3] = xa[q * GP + j][3];
            }
            uint16_t *rowp = &abuf[buf][row * ASTR];
            if constexpr (TWO) {
                // group G = 4hh + qq: pairs (x_p, x_{p+8}); p = 0..3 feed k-step 2qq, p = 4..7 k-step 2qq+1
                const int hh = G >> 2, qq = G & 3;
                uint32_t o[8];
#pragma unroll
                for (int p = 0; p < 8; p += 2) {
                    o[p] = pair_halves<0>(v[4 + p / 2], v[p / 2]);
                    o[p + 1] = pair_halves<1>(v[4 + p / 2], v[p / 2]);
                }
                *reinterpret_cast<u32x4 *>(rowp + 16 * (2 * qq) + 8 * hh) = u32x4{o[0], o[1], o[2], o[3]};
                *reinterpret_cast<u32x4 *>(rowp + 16 * (2 * qq + 1) + 8 * hh) = u32x4{o[4], o[5], o[6], o[7]};
            } else {
                // group G = 2hh + g5: for p = 0..4, r = 0..3: (x[5r+p], x[5r+20+p]) feed k-step 5g5+p
                const int hh = G >> 1, g5 = G & 1;
#pragma unroll
                for (int p = 0; p < 5; ++p) {
                    uint32_t o[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int e = 5 * r + p;   // value index in the group; partner e + 20
                        o[r] = (e & 1) ? pair_halves<1>(v[(e >> 1) + 10], v[e >> 1])
                                       : pair_halves<0>(v[(e >> 1) + 10], v[e >> 1]);
                    }
                    *reinterpret_cast<u32x4 *>(rowp + 16 * (5 * g5 + p) + 8 * hh) = u32x4{o[0], o[1], o[2], o[3]};
                }
            }
        }
    };

    float16_t acc[kMTt][kNT];
#pragma unroll
    for (int mt = 0; mt < kMTt; ++mt)
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) acc[mt][nt] = float16_t{};
    uint32_t bias;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(bias));   // register-held constant (no memory access)

    // 1.6-bit: digit codes of byte pairs (b, b + 4) of each 8-byte half of the lane's 16 bytes
    uint32_t code[kNT][TWO ? 1 : 8];
    auto take_codes = [&](const u32x4 (&wb)[kNT]) {
        if constexpr (!TWO) {
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) {
                    const uint32_t lo = wb[nt][2 * (cc >> 2)], hi = wb[nt][2 * (cc >> 2) + 1];
                    const int sh = 8 * (cc & 3);
                    code[nt][cc] = lut[(lo >> sh) & 0xFFu] | (lut[(hi >> sh) & 0xFFu] << 16);
                }
        }
    };
    // B operand of k-step s, column tile nt (2-bit: from the packed words; 1.6-bit: from the codes)
    auto decode = [&](const u32x4 (&wb)[kNT], int s, int nt) {
        u32x4 b;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if constexpr (TWO)
                b[r] = digits_to_t(wb[nt][s >> 1] >> (2 * (4 * (s & 1) + r)), bias);
            else
                b[r] = digits_to_t(code[nt][4 * (s / 5) + r] >> (2 * (s % 5)), bias);
        }
        return b;
    };

    // Two weight register sets alternate between K tiles (the loop below is unrolled by two so
    // the alternation costs no copies): a tile decodes from one while the next tile's words
    // arrive in the other.  The activations of tile kt + 2 are loaded right after tile kt + 1's
    // are staged, so every load has about one K tile of MFMA work to arrive.
    u32x4 xa[XP];
    u32x4 w0[kNT], w1[kNT];
    // (loads are issued in the loop's order -- activations, then weights -- so the wait
    // counts the compiler derives at the loop entry match those of the loop itself)
    load_a(0, xa);
    load_b(0, w0);
    store_a(0, xa);
    __builtin_amdgcn_sched_barrier(0);
    load_a(1, xa);
    load_b(1, w1);
    __syncthreads();                             // tile 0's activations and the byte table
    take_codes(w0);
    const int aoff = c * ASTR + 8 * h;
    u32x4 afr[kMTt], bop[kNT];
#pragma unroll
    for (int mt = 0; mt < kMTt; ++mt) afr[mt] = *reinterpret_cast<const u32x4 *>(&abuf[0][aoff + 32 * mt * ASTR]);
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) bop[nt] = decode(w0, 0, nt);

    // One K tile: wc holds its weights, wx those of the next tile.  MORE (compile-time, so the
    // tile body has no branches) says whether a next tile exists.
    auto tile = [&](int kt, auto more_tag, u32x4 (&wc)[kNT], u32x4 (&wx)[kNT]) __attribute__((always_inline)) {
        constexpr bool MORE = decltype(more_tag)::value;
        const int buf = kt & 1;
        const uint16_t *acur = &abuf[buf][aoff];
        const uint16_t *anext = &abuf[buf ^ 1][aoff];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            // every wave has stored its share of the next tile (step KS - 2) and read its
            // last operands of this one: the next tile's buffer may be read from here on
            if (MORE && s == KS - 1) __syncthreads();
            u32x4 an[kMTt], bn[kNT];
            if (s + 1 < KS) {
#pragma unroll
                for (int mt = 0; mt < kMTt; ++mt)
                    an[mt] = *reinterpret_cast<const u32x4 *>(acur + 32 * mt * ASTR + 16 * (s + 1));
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) bn[nt] = decode(wc, s + 1, nt);
            } else if (MORE) {
#pragma unroll
                for (int mt = 0; mt < kMTt; ++mt) an[mt] = *reinterpret_cast<const u32x4 *>(anext + 32 * mt * ASTR);
                take_codes(wx);                  // the last decode of this tile's codes was at step KS - 2
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) bn[nt] = decode(wx, 0, nt);
            }
#pragma unroll
            for (int mt = 0; mt < kMTt; ++mt)
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) acc[mt][nt] = mfma32(afr[mt], bop[nt], acc[mt][nt]);
            if (MORE && s == KS - 2) store_a(buf ^ 1, xa);
            // interleave: each MFMA is followed by a share of the next step's decode and reads
#pragma unroll
            for (int i = 0; i < kMTt * kNT; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // 3 VALU
                if (i % 4 == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
            }
            __builtin_amdgcn_sched_barrier(0);
            if (MORE && s == KS - 2) load_a(kt + 2, xa);   // past the last tile: zeros, never stored
            if (MORE && s == KS - 1) load_b(kt + 2, wc);   // wc's last decode was at step KS - 2
            if (s + 1 < KS || MORE) {
#pragma unroll
                for (int mt = 0; mt < kMTt; ++mt) afr[mt] = an[mt];
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) bop[nt] = bn[nt];
            }
        }
    };
    // An even number of tiles keeps a single code path: an odd count gets one more tile past
    // the end, whose activations read as zero, so it adds exact zeros.
    const int KTe = (KT + 1) & ~1;
    for (int kt = 0; kt + 2 < KTe; kt += 2) {
        tile(kt, std::true_type{}, w0, w1);
        tile(kt + 1, std::true_type{}, w1, w0);
    }
    tile(KTe - 2, std::true_type{}, w0, w1);
    tile(KTe - 1, std::false_type{}, w1, w0);

    // epilogue: lane (h, c) holds rows 32mt + 8i + 4h + v of column 32nt + c
#pragma unroll
    for (int mt = 0; mt < kMTt; ++mt)
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

template <int FMT>
static int launch_fmt(const uint16_t *X, const uint8_t *Wp, float scale, int M, int N, int K, int C, uint16_t *Y,
                      hipStream_t s)
{
    const int tiles_m = (M + kBM - 1) / kBM;
    const int tiles_n = (N + kBN - 1) / kBN;
    const int64_t T = (int64_t)tiles_m * tiles_n;
    if (T >= ((int64_t)1 << 30)) return TRI_EINVAL;
    // Few tiles even of 64 rows (a middling M): 64 x 128 workgroups, four per 64 x 512 tile -- no
    // half-empty 128-row tiles, and twice the workgroups of 128-row quarter tiles (30-40% faster
    // where there are at most 64 such tiles; up to 128, two workgroups share a CU and still win
    // a few per cent)
    const int cus = cu_count();
    const int tiles_m64 = (M + 63) / 64;
    const int64_t T64 = (int64_t)tiles_m64 * tiles_n;
    if (T64 <= cus / 2) {
        hipLaunchKernelGGL((k_gemm<FMT, 1, 64>), dim3((unsigned)(4 * T64)), dim3(256), 0, s, X, Wp, scale, M, N, K, C,
                           tiles_m64, tiles_n, 0, Y);
        return hipGetLastError() == hipSuccess ? TRI_OK : TRI_EHIP;
    }
    // A last round of full tiles that would leave more than half of the CUs idle is run as
    // twice as many half-width tiles instead, by a second launch.
    const int r = (int)(T % cus);
    const int tail = (r > 0 && r <= cus / 2) ? r : 0;
    const int full = (int)T - tail;
    if (full > 0)
        hipLaunchKernelGGL((k_gemm<FMT, 4, 128>), dim3((unsigned)full), dim3(256), 0, s, X, Wp, scale, M, N, K, C, tiles_m,
                           tiles_n, 0, Y);
    if (tail > 0)
        hipLaunchKernelGGL((k_gemm<FMT, 2, 128>), dim3((unsigned)(2 * tail)), dim3(256), 0, s, X, Wp, scale, M, N, K, C,
                           tiles_m, tiles_n, full, Y);
    return hipGetLastError() == hipSuccess ? TRI_OK : TRI_EHIP;
}

int launch_gemm(const uint16_t *X, const uint8_t *Wp, float scale, int64_t M, int N, int K, int fmt, uint16_t *Y,
                hipStream_t s)
{
    const int C = (int)(row_bytes(K, fmt) / 16);
    const int64_t S = (int64_t)C * 16;
    // 32-bit buffer offsets: a 128-row activation block and a 128-row weight block must stay
    // below 2^31 bytes, and activations are read in pieces of 8 values (K % 8 == 0).  Other
    // shapes run the small-M kernels over 16-row slices of X.
    const bool fits = (K % 8) == 0 && (int64_t)kBM * K * 2 < ((int64_t)1 << 31) && 128 * S < ((int64_t)1 << 31);
    if (!fits) {
        for (int64_t m0 = 0; m0 < M; m0 += 16) {
            const int mm = (int)((M - m0) < 16 ? (M - m0) : 16);
            const int rc = launch_smallm(X + m0 * K, Wp, scale, mm, N, K, fmt, Y + m0 * N, s);
            if (rc != TRI_OK) return rc;
        }
        return TRI_OK;
    }
    for (int64_t mb = 0; mb < M; mb += (int64_t)1 << 20) {   // keeps the tile count of a launch in int range
        const int mm = (int)((M - mb) < ((int64_t)1 << 20) ? (M - mb) : ((int64_t)1 << 20));
        const int rc = fmt == TRI_FMT_2BIT ? launch_fmt<TRI_FMT_2BIT>(X + mb * K, Wp, scale, mm, N, K, C, Y + mb * N, s)
                                           : launch_fmt<TRI_FMT_1P6BIT>(X + mb * K, Wp, scale, mm, N, K, C, Y + mb * N, s);
        if (rc != TRI_OK) return rc;
    }
    return TRI_OK;
}

}  // namespace tri
