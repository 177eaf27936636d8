// tri_gemm.hip -- ternary linear layer for many activation rows (prefill).
// First version: the MFMA small-M kernel over 16-row slices of X.
#include "tri_device.h"
#include "tri_internal.h"

namespace tri {

int launch_gemm(const uint16_t *X, const uint8_t *Wp, float scale, int64_t M, int N, int K, int fmt, uint16_t *Y,
                hipStream_t s)
{
    for (int64_t m0 = 0; m0 < M; m0 += 16) {
        const int mm = (int)((M - m0) < 16 ? (M - m0) : 16);
        const int rc = launch_smallm(X + m0 * K, Wp, scale, mm, N, K, fmt, Y + m0 * N, s);
        if (rc != TRI_OK) return rc;
    }
    return TRI_OK;
}

}  // namespace tri
