// tri_gemm.hip -- ternary linear layer for many activation rows (prefill) on MFMA.
//
// The layer (Pith review of "Spectra 1.1", "What carries the argument"):
//   Y[m][n] = scale * sum_k t[n][k] * X[m][k],  t in {-1, 0, +1},  fp32 accumulation.
// Here it is a dense contraction (the review's "high-batch" regime), so it runs as a tiled
// fp16 MFMA GEMM (v_mfma_f32_32x32x16_f16) whose B operand is decoded from the packed
// trits in registers -- the gfx950 counterpart of the pages' FP16 x INT2 tensor-core
// kernel with fused dequantisation and asynchronous copies.
//
// Tiling.  A workgroup of 4 waves computes a 128 x 512 tile of Y; wave w owns output
// columns 128w..128w+127 (four 32-column MFMA tiles) for all 128 rows (four 32-row tiles):
// sixteen 32x32 accumulators, 256 accumulation registers.  Every A operand read from LDS
// feeds four MFMAs and every decoded B operand four.  K advances in tiles of one 32-byte
// packed slice per weight row: 128 trits (2-bit, 8 MFMA k-steps of 16) or 160 trits (1.6-bit,
// 10 k-steps).
//  - Order of k: lane half h (lane / 32) of every operand covers the K tile's values
//    KS*8*h ... (KS k-steps), eight consecutive ones per k-step, so an A operand is one
//    16-byte piece of an activation row as it lies in memory.
//  - B (weights): lane (h, c = lane%32) of column tile nt loads bytes 16h..16h+15 of the slice
//    of weight row 32nt + c with one 16-byte buffer load (prefetched one K tile ahead); for
//    1.6-bit, a 256-entry LDS table turns each byte into its five base-3 digits as 2-bit
//    digits (the repeated division b'_i -> x_i that the review's referee report describes for
//    the paper's section 3.2), which are joined into the same 2-bit digit stream.  A k-step
//    takes two bytes of the stream; each byte is copied into both 16-bit halves of a register
//    (v_perm_b32), and two adjacent digits become an exact fp16 pair with one v_and_or_b32
//    and one packed fp16 add (digits_pair).
//  - A (activations): each K tile of the 128 rows is written into one of two LDS buffers by
//    gfx950 buffer loads to LDS (16 bytes per lane, no registers and no LDS write
//    instructions on the way; rows past M and values past K read as zero), one K tile ahead:
//    the analogue of the asynchronous copies of the pages' kernel.  A load instruction reads
//    64 contiguous bytes (four lanes) of each of 16 rows, and the layout in LDS keeps the 16
//    rows that one read pass touches in 16 distinct bank groups.
//  - Software pipeline: the 16 MFMAs of a k-step run while the A and B operands of the next
//    k-step are read and decoded; at the last k-step of a tile every wave waits for its share
//    of the next tile's activations (an explicit vmcnt: the compiler does not wait for what
//    loads to LDS write before a barrier), the single barrier of the tile follows, and the
//    loads of the tile after next are issued into the buffer and the registers just freed.
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

typedef __attribute__((address_space(3))) char *lds_ptr_t;

// s_waitcnt vmcnt(N): at most N vector memory loads of this wave still outstanding (they
// retire in issue order), the other counters not waited for
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | (((N >> 4) & 3) << 14));
}

// Exact fp16 pair (t_a, t_a+1) from two adjacent 2-bit digits of one byte, which `d` holds in
// both 16-bit halves (digit j at bits 2j): the low half keeps digit a in its mantissa, the high
// half digit a + 1, each OR-ed into the power of two 2^e whose mantissa step at that position
// is 1.0 (a = 0: 1024 + d and 256 + d; a = 2: 64 + d and 16 + d), and one packed fp16 add of
// -(2^e + 1) leaves t = d - 1 in each half, exactly.  `bias` holds the two powers of two in a
// vector register, so mask and bias fuse into one v_and_or_b32 (a gfx9 VOP3 instruction takes
// no literal and one scalar operand).
template <int A>
__device__ __forceinline__ uint32_t digits_pair(uint32_t d, uint32_t bias)
{
    static_assert(A == 0 || A == 2, "digit pairs 0-1 and 2-3 of a byte");
    constexpr uint32_t mask = A == 0 ? 0x000C0003u : 0x00C00030u;
    constexpr uint32_t sub = A == 0 ? 0xDC04E401u : 0xCC40D410u;   // (-1025, -257) / (-65, -17)
    const half2_t r = as_h2((d & mask) | bias) + as_h2(sub);
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
    constexpr int PR = BK / 8;                   // 16-byte activation pieces per row and K tile (16 or 20)
    constexpr int NW = TWO ? 4 : 5;              // 32-bit words of 2-bit digits per lane and weight row
    // A buffers, in 16-byte pieces: piece q of tile row r at
    //   (r / 16) 16 PR + (q / 4) 64 + 4 (r % 16) + ((q % 4) ^ ((r % 16) / 4)),
    // so a load instruction fills 64 consecutive positions, a block of 16 rows x 4 pieces whose
    // rows each take 4 consecutive lanes (64 contiguous bytes of the row), and the 16 rows that
    // one LDS read pass touches at one piece fall in 16 distinct bank groups (the XOR).  NI load
    // instructions per wave and tile.  Two separate arrays, not one indexed by a variable: loads
    // to LDS are waited for before LDS reads the compiler cannot prove disjoint from them, and
    // it proves it for distinct arrays.
    constexpr int NI = kBMt * PR / 256;
    static_assert(kBMt * PR % 256 == 0, "whole load instructions per wave");
    __shared__ u32x4 abuf0[kBMt * PR];
    __shared__ u32x4 abuf1[kBMt * PR];
    auto abuf_of = [&](int b) -> u32x4 * { return b ? abuf1 : abuf0; };
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
    const int KTe = (KT + 1) & ~1;               // padded to an even count (see the tile loop)

    // The lane's offset in each of its load instructions at K tile 0 (a tile adds its first
    // value's offset).  Rows past M lie past the buffer and read zeros; pieces past K get an
    // offset past the buffer.  (The out-of-range offset is held in a register: as a literal it
    // would be rebuilt before every select.)  Instruction I of a tile (the wave's i-th) fills
    // rows 16 (I / (PR/4)) + lane / 4, pieces 4 (I % (PR/4)) + ((lane % 4) ^ (lane / 16)).
    uint32_t oob;
    asm volatile("v_mov_b32 %0, 0x80000000" : "=v"(oob));
    auto piece_of = [&](int i) { return 4 * ((wv * NI + i) % (PR / 4)) + ((lane & 3) ^ (lane >> 4)); };
    auto row_of = [&](int i) { return 16 * ((wv * NI + i) / (PR / 4)) + (lane >> 2); };
    uint32_t xoff[NI];
    int klim[NI];                                // the piece's values exist in tiles with k0 < klim
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int row = row_of(i);
        xoff[i] = (uint32_t)(row * K + 8 * piece_of(i)) * 2u;
        klim[i] = K - 8 * piece_of(i);
    }
    // Activations of K tile kt into buffer `buf` (tiles past the end read zeros).  The K test
    // is a per-lane select, not a branch: a branch would split the tile body into blocks, and
    // the compiler then sinks the next tile's first decode below these loads.
    auto load_a = [&](int kt, int buf) {
        const int k0 = kt * BK;                  // wave-uniform
        const lds_ptr_t dst = (lds_ptr_t)(abuf_of(buf) + wv * NI * 64);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint32_t off = k0 < klim[i] ? xoff[i] + 2u * (uint32_t)k0 : oob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, dst + 1024 * i, 16, (int)off, 0, 0, 0);
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

    float16_t acc[kMTt][kNT];
#pragma unroll
    for (int mt = 0; mt < kMTt; ++mt)
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) acc[mt][nt] = float16_t{};
    uint32_t bias01, bias23;                     // register-held constants (no memory access)
    asm volatile("v_mov_b32 %0, 0x5C006400" : "=v"(bias01));
    asm volatile("v_mov_b32 %0, 0x4C005400" : "=v"(bias23));

    // 1.6-bit: the lane's 16 bytes as a stream of 2-bit digits, 80 trits in 5 words (the digits
    // of byte b at bits 10b ...)
    uint32_t str[kNT][TWO ? 1 : NW];
    auto take_codes = [&](const u32x4 (&wb)[kNT]) {
        if constexpr (!TWO) {
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                uint32_t cd[16];
#pragma unroll
                for (int b = 0; b < 16; ++b) cd[b] = lut[(wb[nt][b >> 2] >> (8 * (b & 3))) & 0xFFu];
#pragma unroll
                for (int j = 0; j < NW; ++j) {
                    uint32_t v = 0;
#pragma unroll
                    for (int b = 0; b < 16; ++b) {
                        const int lo = 10 * b - 32 * j;
                        if (lo >= 32 || lo + 10 <= 0) continue;
                        v |= lo >= 0 ? cd[b] << lo : cd[b] >> -lo;
                    }
                    str[nt][j] = v;
                }
            }
        }
    };
    // B operand of k-step s, column tile nt: trits 8s ... 8s+7 of the lane's, bytes 2s and
    // 2s + 1 of its digit stream (2-bit: the packed words themselves)
    auto decode = [&](const u32x4 (&wb)[kNT], int s, int nt) {
        uint32_t w;
        if constexpr (TWO) w = wb[nt][s >> 1];
        else w = str[nt][s >> 1];
        u32x4 b;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const uint32_t sel = (uint32_t)(2 * (s & 1) + e) * 0x00010001u;   // the byte into both halves
            const uint32_t d = perm(w, w, sel);
            b[2 * e] = digits_pair<0>(d, bias01);
            b[2 * e + 1] = digits_pair<2>(d, bias23);
        }
        return b;
    };

    // Loads in flight: the activations and weights of the next tile, issued a tile ahead,
    // activations first (the scheduling barriers keep that order: the waits below count on
    // it).  Tiles 0 and 1 are issued before the loop.
    u32x4 w0[kNT], w1[kNT];
    load_a(0, 0);
    load_a(1, 1);
    __builtin_amdgcn_sched_barrier(0);
    load_b(0, w0);
    load_b(1, w1);
    wait_vm<NI + 2 * kNT>();                     // tile 0's activations
    __syncthreads();                             // every wave's share of them, and the byte table
    take_codes(w0);
    // lane (h, c) reads row 32mt + c, piece KS h + s at step s
    uint32_t aadr[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int q = KS * h + s, r = c & 15;
        aadr[s] = 16u * (uint32_t)((c >> 4) * 16 * PR + (q >> 2) * 64 + 4 * r + ((q & 3) ^ (r >> 2)));
    }
    auto read_a = [&](int buf, int s, int mt) {
        return *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(abuf_of(buf)) + aadr[s] +
                                                16 * 32 * PR * mt);
    };
    u32x4 afr[kMTt], bop[kNT];
#pragma unroll
    for (int mt = 0; mt < kMTt; ++mt) afr[mt] = read_a(0, 0, mt);
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) bop[nt] = decode(w0, 0, nt);

    // One K tile: wc holds its weights, wx those of the next tile.  MORE (compile-time, so the
    // tile body has no branches) says whether a next tile exists.
    auto tile = [&](int kt, auto more_tag, auto buf_tag, u32x4 (&wc)[kNT], u32x4 (&wx)[kNT]) __attribute__((always_inline)) {
        constexpr bool MORE = decltype(more_tag)::value;
        constexpr int buf = decltype(buf_tag)::value;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (MORE && s == KS - 1) {
                // this wave's share of the next tile's activations is in (only the weight
                // loads issued after it may still be in flight) and its reads of this tile are
                // done; after the barrier, every wave's are
                __builtin_amdgcn_s_waitcnt(0x0070 | kNT);   // vmcnt(kNT) lgkmcnt(0)
                __syncthreads();
            }
            u32x4 an[kMTt], bn[kNT];
            if (s + 1 < KS) {
#pragma unroll
                for (int mt = 0; mt < kMTt; ++mt) an[mt] = read_a(buf, s + 1, mt);
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) bn[nt] = decode(wc, s + 1, nt);
            } else if (MORE) {
#pragma unroll
                for (int mt = 0; mt < kMTt; ++mt) an[mt] = read_a(buf ^ 1, 0, mt);
                take_codes(wx);                  // the last decode of this tile's stream was at step KS - 2
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) bn[nt] = decode(wx, 0, nt);
            }
#pragma unroll
            for (int mt = 0; mt < kMTt; ++mt)
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) acc[mt][nt] = mfma32(afr[mt], bop[nt], acc[mt][nt]);
            // interleave: each MFMA is followed by a share of the next step's decode and reads
#pragma unroll
            for (int i = 0; i < kMTt * kNT; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // 3 VALU
                if (i % 4 == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
            }
            __builtin_amdgcn_sched_barrier(0);
            if (MORE && s == KS - 1) {
                // this tile's buffer and weight registers are free: the tile after next
                load_a(kt + 2, buf);
                __builtin_amdgcn_sched_barrier(0);
                load_b(kt + 2, wc);
            }
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
    for (int kt = 0; kt + 2 < KTe; kt += 2) {
        tile(kt, std::true_type{}, std::integral_constant<int, 0>{}, w0, w1);
        tile(kt + 1, std::true_type{}, std::integral_constant<int, 1>{}, w1, w0);
    }
    tile(KTe - 2, std::true_type{}, std::integral_constant<int, 0>{}, w0, w1);
    tile(KTe - 1, std::false_type{}, std::integral_constant<int, 1>{}, w1, w0);
    wait_vm<0>();                                // (the last tile's loads to LDS, past the end, are in)

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
