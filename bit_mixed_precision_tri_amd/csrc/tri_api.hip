// tri_api.hip -- the extern "C" entry points of libtri: argument checks and dispatch.
// Every check runs on the host before any launch; see include/tri.h for the contract.
#include "tri_internal.h"

using namespace tri;
static_assert(TRI_MAX_GROUPS == kMaxGroups, "group table size");

namespace {

bool misaligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }
bool known_fmt(int fmt) { return fmt == TRI_FMT_2BIT || fmt == TRI_FMT_1P6BIT; }
constexpr int64_t kMaxDim = (int64_t)1 << 31;   // K, N and one packed row are indexed with 32-bit ints

int check_pack(const void *W, int64_t N, int64_t K, const void *Wp)
{
    if (!W || !Wp || N < 1 || K < 1 || N >= kMaxDim || K >= kMaxDim) return TRI_EINVAL;
    if (misaligned(Wp)) return TRI_EALIGN;
    return TRI_OK;
}

int check_linear(const void *X, const void *Wp, int64_t M, int64_t N, int64_t K, int fmt, const void *Y)
{
    if (!X || !Wp || !Y || M < 1 || N < 1 || K < 1 || !known_fmt(fmt)) return TRI_EINVAL;
    if (N >= kMaxDim || K >= kMaxDim || M >= kMaxDim) return TRI_EINVAL;
    if (misaligned(X) || misaligned(Wp) || misaligned(Y)) return TRI_EALIGN;
    return TRI_OK;
}

// The kernel family for a shape.  Up to 16 rows, the small-M kernels (at M = 1 the MFMA kernel
// beats the VALU GEMV).  Above, the small-M kernels take one pass over the weights per 16-row
// slice of X, while the GEMM's parallelism comes from its output tiles alone, so with few tiles
// most CUs idle.  Both costs per unit of K, from fits to measured times on MI355X (M = 17 .. 768;
// K x N = 4096 x 4096, 4096 x 11008, 11008 x 4096, 8192 x 28672, 28672 x 8192; both formats):
//   small-M  ceil(M/16) * N * c,  c = 0.10 ps (2-bit) / 0.127 ps (1.6-bit) per trit and slice;
//            rows past eight steps per wave 1.6x / 1.2x that, rows past sixteen (the streaming
//            kernel) 5x / 1.9x;
//   GEMM     with T64 = ceil(M/64) * ceil(N/512) tiles of 64 rows: at most 64 of them, one round
//            of 64 x 128 workgroups, 4.8 ns (2-bit) / 6.3 ns (1.6-bit); at most 128, 8.8 / 10.7
//            ns; beyond, u * R with u = 13 / 16 ns per round of 128 x 256 workgroups and R the
//            rounds of the launch of 128-row tiles (a last round of at most 128 tiles runs at half
//            width).
int select_algo(int64_t M, int64_t N, int64_t K, int fmt)
{
    if (M <= 16) return TRI_ALGO_SMALLM;
    const int64_t cus = cu_count();
    const bool two = fmt == TRI_FMT_2BIT;
    double c = two ? 0.10 : 0.127;               // ps
    if (K > (two ? 32768 : 35840)) c *= two ? 5.0 : 1.9;
    else if (K > (two ? 16384 : 20480)) c *= two ? 1.6 : 1.2;
    const int64_t tn = (N + 511) / 512;
    const int64_t T64 = ((M + 63) / 64) * tn, T = ((M + 127) / 128) * tn;
    const int64_t r = T % cus;
    const int64_t R = (r > 0 && r <= cus / 2) ? 2 * (T / cus) + 1 : 2 * ((T + cus - 1) / cus);
    const double small = (double)((M + 15) / 16) * (double)N * c;
    const double gemm = T64 <= cus / 4 ? (two ? 4800.0 : 6300.0)
                      : T64 <= cus / 2 ? (two ? 8800.0 : 10700.0)
                                        : (two ? 13000.0 : 16000.0) * (double)R;
    return small < gemm ? TRI_ALGO_SMALLM : TRI_ALGO_GEMM;
}

int run_linear(const _Float16 *X, const uint8_t *Wp, float scale, int64_t M, int64_t N, int64_t K, int fmt,
               _Float16 *Y, int algo, hipStream_t s)
{
    const uint16_t *x = reinterpret_cast<const uint16_t *>(X);
    uint16_t *y = reinterpret_cast<uint16_t *>(Y);
    switch (algo) {
    case TRI_ALGO_GEMV:
        if (M != 1 || fmt != TRI_FMT_2BIT) return TRI_EINVAL;
        return launch_gemv2(x, Wp, scale, (int)N, (int)K, y, s);
    case TRI_ALGO_SMALLM:
        if (M > 16) {
            // one launch over 16-row slices of X where the batched kernel serves the shape,
            // else one small-M call per slice
            int n = (int)N;
            const Groups gr = make_groups(1, &Wp, &scale, &n, &y);
            if (launch_mvm(x, gr, (int)M, (int)K, fmt, s)) return hipGetLastError() == hipSuccess ? TRI_OK : TRI_EHIP;
            for (int64_t m0 = 0; m0 < M; m0 += 16) {
                const int64_t mm = (M - m0) < 16 ? (M - m0) : 16;
                const int rc = run_linear(X + m0 * K, Wp, scale, mm, N, K, fmt, Y + m0 * N, TRI_ALGO_SMALLM, s);
                if (rc != TRI_OK) return rc;
            }
            return TRI_OK;
        }
        if (launch_decode(x, Wp, scale, (int)M, (int)N, (int)K, fmt, y, s))
            return hipGetLastError() == hipSuccess ? TRI_OK : TRI_EHIP;
        return launch_smallm(x, Wp, scale, (int)M, (int)N, (int)K, fmt, y, s);   // long rows: streaming variant
    case TRI_ALGO_GEMM:
        return launch_gemm(x, Wp, scale, M, (int)N, (int)K, fmt, y, s);
    default:
        return TRI_EINVAL;
    }
}

}  // namespace

int tri::cu_count()
{
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < kMaxDevices) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return 256;
    if (dev >= 0 && dev < kMaxDevices) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

extern "C" {

int64_t tri_row_bytes(int64_t K, int fmt) { return row_bytes(K, fmt); }

int64_t tri_quantize_workspace_bytes(int64_t N, int64_t K)
{
    if (N < 1 || K < 1 || N >= kMaxDim || K >= kMaxDim) return -1;
    return quant_workspace_bytes(N * K);
}

int tri_quantize(const float *W, int64_t N, int64_t K, int fmt, uint8_t *Wp, float *scale_out, void *workspace,
                 int64_t workspace_bytes, hipStream_t stream)
{
    if (!W || !Wp || !scale_out || !workspace || !known_fmt(fmt)) return TRI_EINVAL;
    if (N < 1 || K < 1 || N >= kMaxDim || K >= kMaxDim) return TRI_EINVAL;
    if (workspace_bytes < quant_workspace_bytes(N * K)) return TRI_EINVAL;
    if (misaligned(W) || misaligned(Wp) || misaligned(workspace) || (reinterpret_cast<uintptr_t>(scale_out) & 3u))
        return TRI_EALIGN;
    return launch_quantize(W, N, K, fmt, Wp, scale_out, workspace, stream);
}

int tri_quantize_noalloc(const float *W, int64_t N, int64_t K, int fmt, uint8_t *Wp, float *scale_out,
                         hipStream_t stream)
{
    if (!W || !Wp || !scale_out || !known_fmt(fmt)) return TRI_EINVAL;
    if (N < 1 || K < 1 || N >= kMaxDim || K >= kMaxDim) return TRI_EINVAL;
    if (quant_workspace_bytes(N * K) > quant_scratch_bytes()) return TRI_EINVAL;
    if (misaligned(W) || misaligned(Wp) || (reinterpret_cast<uintptr_t>(scale_out) & 3u)) return TRI_EALIGN;
    void *ws = quant_scratch();
    if (!ws) return TRI_EHIP;
    return launch_quantize(W, N, K, fmt, Wp, scale_out, ws, stream);
}

int tri_pack2(const int8_t *W, int64_t N, int64_t K, uint8_t *Wp, hipStream_t stream)
{
    const int rc = check_pack(W, N, K, Wp);
    return rc != TRI_OK ? rc : launch_pack(W, N, K, TRI_FMT_2BIT, Wp, stream);
}

int tri_pack16(const int8_t *W, int64_t N, int64_t K, uint8_t *Wp, hipStream_t stream)
{
    const int rc = check_pack(W, N, K, Wp);
    return rc != TRI_OK ? rc : launch_pack(W, N, K, TRI_FMT_1P6BIT, Wp, stream);
}

int tri_unpack(const uint8_t *Wp, int64_t N, int64_t K, int fmt, int8_t *W, hipStream_t stream)
{
    if (!known_fmt(fmt)) return TRI_EINVAL;
    const int rc = check_pack(W, N, K, Wp);
    return rc != TRI_OK ? rc : launch_unpack(Wp, N, K, fmt, W, stream);
}

int tri_select_algo(int64_t M, int64_t N, int64_t K, int fmt)
{
    if (M < 1 || N < 1 || K < 1 || !known_fmt(fmt) || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return TRI_EINVAL;
    return select_algo(M, N, K, fmt);
}

int tri_linear(const _Float16 *X, const uint8_t *Wp, float scale, int64_t M, int64_t N, int64_t K, int fmt,
               _Float16 *Y, hipStream_t stream)
{
    const int rc = check_linear(X, Wp, M, N, K, fmt, Y);
    return rc != TRI_OK ? rc : run_linear(X, Wp, scale, M, N, K, fmt, Y, select_algo(M, N, K, fmt), stream);
}

int tri_linear_algo(const _Float16 *X, const uint8_t *Wp, float scale, int64_t M, int64_t N, int64_t K, int fmt,
                    _Float16 *Y, int algo, hipStream_t stream)
{
    const int rc = check_linear(X, Wp, M, N, K, fmt, Y);
    if (rc != TRI_OK) return rc;
    if (algo == TRI_ALGO_AUTO) algo = select_algo(M, N, K, fmt);
    return run_linear(X, Wp, scale, M, N, K, fmt, Y, algo, stream);
}

int tri_linear_grouped(const _Float16 *X, const uint8_t *const *Wp, const float *scale, int64_t M, const int64_t *N,
                       int64_t K, int fmt, _Float16 *const *Y, int G, hipStream_t stream)
{
    if (!Wp || !scale || !N || !Y || G < 1 || G > TRI_MAX_GROUPS) return TRI_EINVAL;
    for (int g = 0; g < G; ++g) {
        const int rc = check_linear(X, Wp[g], M, N[g], K, fmt, Y[g]);
        if (rc != TRI_OK) return rc;
    }
    int64_t blocks = 0;
    for (int g = 0; g < G; ++g) blocks += (N[g] + 15) / 16;
    if (blocks >= ((int64_t)1 << 31)) return TRI_EINVAL;
    const uint16_t *x = reinterpret_cast<const uint16_t *>(X);
    bool small = true;                           // every matrix on the small-M kernels
    for (int g = 0; g < G; ++g) small = small && select_algo(M, N[g], K, fmt) == TRI_ALGO_SMALLM;
    if (small) {
        int n[kMaxGroups];
        uint16_t *y[kMaxGroups];
        for (int g = 0; g < G; ++g) {
            n[g] = (int)N[g];
            y[g] = reinterpret_cast<uint16_t *>(Y[g]);
        }
        const Groups gr = make_groups(G, Wp, scale, n, y);
        const bool done = M == 1 ? launch_mv1(x, gr, (int)K, fmt, stream)
                          : (M <= 4 && launch_mvr(x, gr, (int)M, (int)K, fmt, stream)) ||
                                launch_mvm(x, gr, (int)M, (int)K, fmt, stream);
        if (done) return hipGetLastError() == hipSuccess ? TRI_OK : TRI_EHIP;
    }
    // shapes outside the grouped kernels' range: one call per matrix
    for (int g = 0; g < G; ++g) {
        const int rc = run_linear(X, Wp[g], scale[g], M, N[g], K, fmt, Y[g], select_algo(M, N[g], K, fmt), stream);
        if (rc != TRI_OK) return rc;
    }
    return TRI_OK;
}

int tri_linear_fused(const _Float16 *X, const uint8_t *const *Wp, const float *scale, int64_t M, const int64_t *N,
                     int64_t K, int fmt, _Float16 *const *Y, int G, const tri_glue *glue, hipStream_t stream)
{
    if (!glue || !Wp || !scale || !N || !Y || G < 1 || G > TRI_MAX_GROUPS) return TRI_EINVAL;
    const bool pair = glue->pair != 0;
    if (pair && (G != 2 || N[0] != N[1])) return TRI_EINVAL;
    for (int g = 0; g < G; ++g) {
        const int rc = check_linear(X, Wp[g], M, N[g], K, fmt, (pair && g == 1) ? Y[0] : Y[g]);
        if (rc != TRI_OK) return rc;
    }
    if (M > 16 || (K % 8) != 0) return TRI_EINVAL;
    if ((glue->norm || pair) && K > (fmt == TRI_FMT_2BIT ? 16384 : 20480)) return TRI_EINVAL;
    int64_t blocks = 0;
    for (int g = 0; g < G; ++g) blocks += (N[g] + 15) / 16;
    if (blocks >= ((int64_t)1 << 31)) return TRI_EINVAL;
    if (glue->norm && !(glue->norm_eps >= 0.f && glue->norm_eps <= 3.4e38f)) return TRI_EINVAL;   // (NaN fails)
    if (misaligned(glue->norm_gain)) return TRI_EALIGN;
    Fusion fu{};
    fu.gain = glue->norm ? reinterpret_cast<const uint16_t *>(glue->norm_gain) : nullptr;
    fu.norm = glue->norm ? 1 : 0;
    fu.eps = glue->norm_eps;
    fu.pair = pair ? 1 : 0;
    for (int g = 0; g < G; ++g) {
        const _Float16 *r = glue->residual ? glue->residual[g] : nullptr;
        if (pair && g == 1 && r) return TRI_EINVAL;
        if (misaligned(r)) return TRI_EALIGN;
        fu.res[g] = reinterpret_cast<const uint16_t *>(r);
    }
    int n[kMaxGroups];
    uint16_t *y[kMaxGroups];
    for (int g = 0; g < G; ++g) {
        n[g] = (int)N[g];
        y[g] = reinterpret_cast<uint16_t *>(Y[g]);
    }
    Groups gr = make_groups(G, Wp, scale, n, y);
    if (pair) gr.blk[2] = gr.blk[1];            // the grid covers matrix 0's rows; each workgroup reads both
    const uint16_t *x = reinterpret_cast<const uint16_t *>(X);
    const bool done =
        M == 1 ? launch_mv1(x, gr, (int)K, fmt, stream, &fu)
               : (M <= 4 && launch_mvr(x, gr, (int)M, (int)K, fmt, stream, &fu)) ||
                     launch_mvm(x, gr, (int)M, (int)K, fmt, stream, &fu);
    if (!done) return TRI_EINVAL;                // a shape the glue variants do not serve
    return hipGetLastError() == hipSuccess ? TRI_OK : TRI_EHIP;
}

const char *tri_status_string(int code)
{
    switch (code) {
    case TRI_OK: return "ok";
    case TRI_EINVAL: return "invalid argument";
    case TRI_EALIGN: return "pointer not 16-byte aligned";
    case TRI_EHIP: return "HIP launch error";
    default: return "unknown status";
    }
}

int tri_probe_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t stream)
{
    if (!src || !sink || bytes < 16 || (bytes % 16) != 0) return TRI_EINVAL;
    if (misaligned(src)) return TRI_EALIGN;
    return launch_probe_read(src, bytes, sink, stream);
}

int tri_probe_copy(const void *src, void *dst, int64_t bytes, hipStream_t stream)
{
    if (!src || !dst || bytes < 16 || (bytes % 16) != 0) return TRI_EINVAL;
    if (misaligned(src) || misaligned(dst)) return TRI_EALIGN;
    return launch_probe_copy(src, dst, bytes, stream);
}

int tri_probe_empty(int64_t workgroups, int threads, uint32_t *sink, hipStream_t stream)
{
    if (!sink || workgroups < 1 || workgroups >= kMaxDim || threads < 64 || threads > 1024 || (threads % 64) != 0)
        return TRI_EINVAL;
    return launch_probe_empty(workgroups, threads, sink, stream);
}

int tri_probe_rows(const _Float16 *X, const uint8_t *Wp, int64_t N, int64_t K, int fmt, int waves, _Float16 *Y,
                   hipStream_t stream)
{
    if (!X || !Wp || !Y || N < 1 || K < 1 || N >= kMaxDim || K >= kMaxDim || !known_fmt(fmt)) return TRI_EINVAL;
    if (waves != 4 && waves != 8) return TRI_EINVAL;
    if ((row_bytes(K, fmt) / 16 + 4 * waves - 1) / (4 * waves) > 8 || N * row_bytes(K, fmt) >= kMaxDim)
        return TRI_EINVAL;
    if (misaligned(X) || misaligned(Wp)) return TRI_EALIGN;
    return launch_probe_rows(reinterpret_cast<const uint16_t *>(X), Wp, (int)N, (int)K, fmt, waves,
                             reinterpret_cast<uint16_t *>(Y), stream);
}

int tri_probe_stream(const void *src, int64_t bytes, int workgroups, int unroll, uint32_t *sink, hipStream_t stream)
{
    if (!src || !sink || bytes < 16 || (bytes % 16) != 0 || bytes >= kMaxDim || workgroups < 1) return TRI_EINVAL;
    if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) return TRI_EINVAL;
    if (misaligned(src)) return TRI_EALIGN;
    return launch_probe_stream(src, bytes, workgroups, unroll, sink, stream);
}

}  // extern "C"
