// w4_mfma.hip -- prefill-shaped W4A16 GEMM on the matrix cores (placeholder
// until the tile is written: every call reports W4_ERR_UNSUPPORTED).
#include <cstdio>

#include "w4_dispatch.h"

namespace w4 {

int launch_mfma_gemm(const void*, int, int, int, int, const uint16_t*, int, void*, int,
                     int, hipStream_t) {
    return fail(W4_ERR_UNSUPPORTED, "gemm: matrix-core tile not built");
}

void describe_mfma(int M, int N, int K, int group, char* buf, size_t len) {
    snprintf(buf, len, "mfma (not built) M=%d N=%d K=%d g=%d", M, N, K, group);
}

}  // namespace w4
