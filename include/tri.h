/*
 * tri.h -- C ABI of libtri, the gfx950 (MI355X) ternary linear layer.
 *
 * The layer (Pith review of "Spectra 1.1: Scaling Laws and Efficient Inference
 * for Ternary Language Models", section "What carries the argument"): a weight
 * matrix W with entries in {-1, 0, +1} times one shared floating-point scale,
 * applied to fp16 activations,
 *
 *     Y[m][n] = fp16_rne( scale * sum_k W[n][k] * X[m][k] ),   accumulated in fp32.
 *
 * Weights are stored losslessly in one of two packings (same review, "Core
 * claim" and "What carries the argument": 2^p > 3^k, so 5 trits fit in 8 bits):
 *
 *   TRI_FMT_2BIT    base-4: byte = sum_{j<4} (t[4b+j] + 1) * 4^j
 *                   (trit 4b+j in bits 2j..2j+1; digit 3 never produced)
 *   TRI_FMT_1P6BIT  base-3: byte = sum_{j<5} (t[5b+j] + 1) * 3^j   (0..242)
 *
 * Layout of a packed matrix: N rows (output features) one after another, each
 * tri_row_bytes(K, fmt) bytes long; a row is padded with zero trits to a
 * multiple of 64 trits (2-bit) or 80 trits (1.6-bit), so every row is a whole
 * number of 16-byte chunks and starts 16-byte aligned.
 *
 * Conventions for every call:
 *  - All array pointers are DEVICE pointers owned by the caller.  The library
 *    allocates no memory.  The only state it keeps is, per device, the compute
 *    unit count and the resident workgroups of a few kernel variants, each
 *    queried from the HIP runtime once and never changed; calls are thread-safe
 *    and deterministic (no atomics; the reduction order is fixed).
 *  - Work is enqueued asynchronously on `stream` (0 = the null stream).  A
 *    device fault surfaces at the caller's next synchronisation.
 *  - Argument checks run on the host before anything is launched; on failure
 *    nothing is launched and a negative status is returned.
 *  - Outputs must not alias inputs.
 */
#ifndef TRI_H
#define TRI_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { TRI_FMT_2BIT = 0, TRI_FMT_1P6BIT = 1 };

enum {
    TRI_OK = 0,
    TRI_EINVAL = -1,   /* a size < 1 (or too large), a null pointer, an unknown format or algorithm */
    TRI_EALIGN = -2,   /* a pointer that must be 16-byte aligned is not */
    TRI_EHIP = -3      /* the HIP runtime reported an error at launch */
};

/* Kernel families of tri_linear (see tri_linear_algo). */
enum {
    TRI_ALGO_AUTO = 0,     /* pick from (M, fmt): the default of tri_linear */
    TRI_ALGO_GEMV = 1,     /* M == 1, 2-bit only: VALU dot products, lanes own K-slices */
    TRI_ALGO_SMALLM = 2,   /* any M, in 16-row slices of X: MFMA 16x16x32 f16 with trits decoded
                              in registers, one pass over the weights per slice (the choice up to
                              M = 16, M = 1 included, and above while the GEMM has too few tiles
                              to fill the chip) */
    TRI_ALGO_GEMM = 3      /* any M: tiled MFMA 32x32x16 f16 GEMM, activations staged in LDS and
                              trits decoded in registers (prefill) */
};

/* Bytes of one packed row of K trits: 16*ceil(K/64) (2-bit) or 16*ceil(K/80)
 * (1.6-bit).  The densities are the pages' (Pith review, "Core claim": base-4 and
 * base-3 encodings; "What carries the argument": 5 trits in 8 bits since
 * 3^5 < 2^8); the row padding is this library's reading of a layout the pages
 * leave open: every row is padded with zero trits to whole 16-byte chunks (64
 * trits in 2-bit, 80 in 1.6-bit), so a row starts 16-byte aligned and is read
 * with 16-byte loads.  At K a multiple of 64 the 2-bit row is exactly K/4 bytes;
 * a 1.6-bit row exceeds ceil(K/5) by at most 15 bytes.
 * Returns -1 if K < 1 or fmt is unknown; pure host arithmetic, launches nothing. */
int64_t tri_row_bytes(int64_t K, int fmt);

/* 2-bit packing (Pith review, "Core claim": base-4 encoding).
 * W: N*K int8, row-major (row n = output feature n).  Any int8 is accepted and
 * sign(w) is encoded.  Wp: N*tri_row_bytes(K, TRI_FMT_2BIT) bytes, 16-byte aligned.
 * Errors: TRI_EINVAL (N < 1, K < 1, null), TRI_EALIGN (Wp), TRI_EHIP. */
int tri_pack2(const int8_t *W, int64_t N, int64_t K, uint8_t *Wp, hipStream_t stream);

/* 1.6-bit packing (Pith review, "What carries the argument": 3^5 = 243 < 2^8,
 * 1.6 bits per weight; "Core claim": base-3 encoding).  Same arguments as
 * tri_pack2 with rows of tri_row_bytes(K, TRI_FMT_1P6BIT) bytes. */
int tri_pack16(const int8_t *W, int64_t N, int64_t K, uint8_t *Wp, hipStream_t stream);

/* Unpack (Pith review, "Significance": the packing correctness theorem of the
 * paper's Appendix E; "Referee Report" minor comment 5: the 1.6-bit decode is
 * the repeated-division sequence b'_i -> x_i).  Defined for every byte value:
 * a 2-bit code 3 gives 0, and 1.6-bit bytes 243..255 go through the same
 * repeated division by 3 (five digits).  Writes the first K trits of each row.
 * Wp: N rows of tri_row_bytes(K, fmt) bytes, 16-byte aligned; W: N*K int8.
 * Errors: TRI_EINVAL, TRI_EALIGN (Wp), TRI_EHIP. */
int tri_unpack(const uint8_t *Wp, int64_t N, int64_t K, int fmt, int8_t *W, hipStream_t stream);

/* Workspace (device bytes, a multiple of 8) that tri_quantize needs for an N x K
 * matrix; -1 if N or K is < 1 or >= 2^31.  It depends on N*K only. */
int64_t tri_quantize_workspace_bytes(int64_t N, int64_t K);

/* Quantise latent full-precision weights to trits and one scale, and pack them
 * (Pith review, "What carries the argument": latent full-precision weights rounded
 * on the fly to {-1,0,1} times one shared scale; the review's domain assumptions:
 * round-to-nearest).  The pages do not give the scale rule; the one taken is
 *     scale = float32( sum_{n,k} |W[n][k]| / (N*K) )   (summed in float64),
 *     t     = round_half_to_even(W / scale) clipped to [-1, 1]; 0 when scale == 0,
 * so a weight becomes sign(w) exactly when 2|w| > scale, ties giving 0.
 * W: N*K float32 row-major, 16-byte aligned, finite (non-finite weights give an
 * unspecified scale and trits).  Wp: N*tri_row_bytes(K, fmt) bytes, 16-byte
 * aligned, written as tri_pack2 / tri_pack16 would pack the trits.  scale_out: one
 * float, 4-byte aligned, written on the stream (read it after synchronising).
 * workspace: at least tri_quantize_workspace_bytes(N, K) bytes, 16-byte aligned,
 * owned by the caller, overwritten; calls that share a workspace must be ordered
 * on one stream.  W must not alias Wp, scale_out or workspace.
 * Errors: TRI_EINVAL (a size < 1 or >= 2^31, null, unknown fmt, workspace too
 * small), TRI_EALIGN, TRI_EHIP. */
int tri_quantize(const float *W, int64_t N, int64_t K, int fmt, uint8_t *Wp, float *scale_out,
                 void *workspace, int64_t workspace_bytes, hipStream_t stream);

/* tri_quantize for callers that cannot allocate device memory or pass a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same launches and results, with the partial sums kept in a
 * static device array of the library (16 KB per device, TRI_QUANTIZE_SCRATCH_BYTES,
 * held until the process ends), so the call allocates nothing.  The array is
 * enough for every N x K (at most 2048 partial sums); a matrix needing more is
 * rejected with TRI_EINVAL.  Every call on one device shares that device's array
 * and overwrites it (nothing in it needs to start at zero): calls that may overlap
 * on one device (several streams, several threads) race and must be ordered by the
 * caller.  Arguments and errors as tri_quantize without the workspace; TRI_EHIP also
 * if the array's device address cannot be obtained. */
enum { TRI_QUANTIZE_SCRATCH_BYTES = 16384 };
int tri_quantize_noalloc(const float *W, int64_t N, int64_t K, int fmt, uint8_t *Wp, float *scale_out,
                         hipStream_t stream);

/* The ternary linear layer (Pith review, "What carries the argument"):
 *   Y[m][n] = fp16_rne(scale * sum_k t[n][k] * X[m][k]), fp32 accumulation.
 * X: M*K fp16 row-major (row stride K); Wp: packed weights as above; Y: M*N fp16
 * row-major.  X, Wp and Y must be 16-byte aligned.  scale is any finite fp32.
 * Wp must hold bytes produced by tri_pack2 / tri_pack16 for this K (2-bit code
 * 3 and 1.6-bit bytes above 242 give unspecified, finite results).  X is
 * expected finite (a non-finite x may give NaN in every output it touches).
 * Errors: TRI_EINVAL (a size < 1, K or N >= 2^31, null, unknown fmt),
 * TRI_EALIGN, TRI_EHIP. */
int tri_linear(const _Float16 *X, const uint8_t *Wp, float scale,
               int64_t M, int64_t N, int64_t K, int fmt, _Float16 *Y, hipStream_t stream);

/* tri_linear with the kernel family chosen by the caller (for measurement and
 * tests).  TRI_ALGO_GEMV needs M == 1 and TRI_FMT_2BIT, else TRI_EINVAL.  Results of every family satisfy the same
 * error bound; they are not bitwise equal to one another. */
int tri_linear_algo(const _Float16 *X, const uint8_t *Wp, float scale,
                    int64_t M, int64_t N, int64_t K, int fmt, _Float16 *Y,
                    int algo, hipStream_t stream);

/* Several ternary linear layers that read the same activations, in one launch (for
 * example the Q, K and V projections of a block, or its gate and up projections): for
 * g < G,  Y[g] = fp16_rne(scale[g] * X W_g^T)  with W_g of N[g] rows packed for this K and
 * fmt, exactly as tri_linear would compute each one.  Wp, scale, N and Y are HOST arrays of
 * G entries (the pointers they hold are device pointers, with tri_linear's alignment and
 * aliasing rules); 1 <= G <= TRI_MAX_GROUPS.  Where tri_linear would pick TRI_ALGO_SMALLM for
 * every matrix, one launch serves all G (the launch's fixed cost is paid once); other shapes
 * run one call per matrix.
 * Errors: those of tri_linear for any matrix, TRI_EINVAL for a bad G or a null array. */
enum { TRI_MAX_GROUPS = 4 };
int tri_linear_grouped(const _Float16 *X, const uint8_t *const *Wp, const float *scale, int64_t M,
                       const int64_t *N, int64_t K, int fmt, _Float16 *const *Y, int G,
                       hipStream_t stream);

/* The glue of a decode block folded into a grouped layer (tri_linear_fused).  The
 * pages name the parts of a block, not this placement (Pith review, "If this is
 * right": the end-to-end speed-up trails the layer's because of the work outside
 * the linear layers). */
typedef struct {
    const _Float16 *norm_gain;         /* K fp16, or NULL for a gain of 1 */
    int norm;                          /* non-zero: RMS-normalise each input row:
                                          x * gain / sqrt(mean_k(x^2) + norm_eps) */
    float norm_eps;                    /* >= 0 and finite */
    int pair;                          /* non-zero: G == 2 and N[0] == N[1]; matrices 0 and 1
                                          are the gate and up projections of a gated MLP and
                                          only Y[0] = fp16(silu(y0) * y1) is written, with
                                          silu(z) = z / (1 + e^-z) (Y[1] may be NULL) */
    const _Float16 *const *residual;   /* NULL, or a HOST array of G pointers, each NULL or an
                                          M*N[g] fp16 residual added before rounding (it may
                                          be Y[g] itself: an in-place residual add); with
                                          pair, residual[1] must be NULL */
} tri_glue;

/* tri_linear_grouped with the glue: for g < G (g = 0 only with pair),
 *   y_g  = scale[g] * (x' W_g^T),  x' = rmsnorm(X) if norm, else X;
 *   Y[g] = fp16_rne( residual[g] + (pair ? silu(y_0) * y_1 : y_g) ).
 * The y_g are fp32 (never rounded on their own); the gained activations are
 * rounded to fp16 as an unfused RMSNorm output would be.  Served by the small-M
 * kernels in one launch for all G matrices; needs M <= 16 and K % 8 == 0.  With
 * norm or pair, K <= 16384 (2-bit) or K <= 20480 (1.6-bit), and for M > 8 also
 * K <= 15360 (1.6-bit with norm) and K <= 8192 / 10240 (2-bit / 1.6-bit with
 * pair); with neither, the row limits of tri_linear's MFMA small-M kernels apply
 * (K <= 16384 / 20480 at least).  Other shapes are rejected with TRI_EINVAL
 * before anything is launched.  norm_gain and the residuals must be 16-byte aligned
 * device pointers and must not alias Wp or (except residual[g] == Y[g]) any Y.
 * Errors: those of tri_linear_grouped, TRI_EINVAL for a null glue, a bad eps, a
 * bad pair or a shape outside the range above, TRI_EALIGN. */
int tri_linear_fused(const _Float16 *X, const uint8_t *const *Wp, const float *scale, int64_t M,
                     const int64_t *N, int64_t K, int fmt, _Float16 *const *Y, int G,
                     const tri_glue *glue, hipStream_t stream);

/* The algorithm tri_linear would pick for (M, N, K, fmt); TRI_EINVAL if invalid.  Up to
 * M = 16 it is TRI_ALGO_SMALLM; above, whichever of TRI_ALGO_SMALLM and TRI_ALGO_GEMM a cost
 * model fitted to MI355X timings says is faster (the small-M kernels' time grows with the
 * number of 16-row slices; the GEMM's is flat while its 64 x 512 tiles fill at most half the
 * CUs, then grows with its rounds of 128 x 512 tiles). */
int tri_select_algo(int64_t M, int64_t N, int64_t K, int fmt);

/* Human-readable name of a status code (static string, never NULL). */
const char *tri_status_string(int code);

/* ---- Measurement aids (not part of the layer) ----------------------------
 * tri_probe_read streams `bytes` bytes (a multiple of 16, 16-byte aligned) with
 * 16-byte loads and writes one word to `sink` (4 bytes) only if a
 * data-dependent test that practically never holds passes; it is the
 * size-matched read floor for the weight stream.  tri_probe_copy copies
 * `bytes` bytes (a multiple of 16, both 16-byte aligned) from src to dst; it
 * calibrates hardware byte counters.  Errors: TRI_EINVAL, TRI_EALIGN, TRI_EHIP. */
int tri_probe_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t stream);
int tri_probe_copy(const void *src, void *dst, int64_t bytes, hipStream_t stream);

/* Launch-cost and read-pattern probes of the decode floor (measurement aids).
 * tri_probe_empty launches an empty kernel of `workgroups` workgroups of
 * `threads` threads (64..1024, a multiple of 64); sink (4 bytes) is never written.
 * tri_probe_rows issues exactly the loads of the one-row decode kernel over an N x
 * tri_row_bytes(K, fmt) packed matrix and a K-wide fp16 row X (16 rows per
 * workgroup of `waves` = 4 or 8 waves, the same chunk of every lane and the same
 * whole-line activation loads) and nothing else: it writes one 16-bit word per
 * matrix row to Y (N fp16 slots) that folds the bytes it read; rows longer than 8
 * steps of 4 chunks per wave give TRI_EINVAL.  tri_probe_stream reads `bytes`
 * bytes (a multiple of 16, below 2^31) with a grid of `workgroups` workgroups of
 * 256 threads, each lane keeping `unroll` (1, 2, 4 or 8) 16-byte loads in flight
 * per round; sink is written only if a data-dependent test that practically never
 * holds passes.  Errors: TRI_EINVAL, TRI_EALIGN (X, Wp, src), TRI_EHIP. */
int tri_probe_empty(int64_t workgroups, int threads, uint32_t *sink, hipStream_t stream);
int tri_probe_rows(const _Float16 *X, const uint8_t *Wp, int64_t N, int64_t K, int fmt, int waves,
                   _Float16 *Y, hipStream_t stream);
int tri_probe_stream(const void *src, int64_t bytes, int workgroups, int unroll, uint32_t *sink,
                     hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TRI_H */
