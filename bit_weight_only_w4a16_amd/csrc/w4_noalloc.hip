// w4_noalloc.hip -- w4a16_gemm for callers that cannot allocate memory
// (code under graph capture, tight serving loops, harnesses that forbid
// hipMalloc): the run-time transform's output goes to a fixed device array
// of this library instead of a caller workspace.
//
// The array is a file-scope __device__ variable, so each GPU holds its own
// copy at its own address from module load until the process ends.  Host
// code never passes the variable's name to a kernel (on the host that name
// is only a stand-in): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept per device.
#include <mutex>

#include "w4_dispatch.h"

namespace w4 {

constexpr size_t kScratchBytes = size_t(8) << 20;   // 8 MiB: M * K * 2 bytes
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// The calling thread's current device's copy of `scratch`.
static int scratch_ptr(void** out) {
    int dev = 0;
    int st = hip_fail(hipGetDevice(&dev), "hipGetDevice");
    if (st != W4_OK) return st;
    if (dev < 0 || dev >= kMaxDevices)
        return fail(W4_ERR_UNSUPPORTED, "gemm_noalloc: device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        st = hip_fail(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (st != W4_OK) return st;
        if (!p) return fail(W4_ERR_HIP, "gemm_noalloc: scratch has no device address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return W4_OK;
}

}  // namespace w4

using namespace w4;

extern "C" {

size_t w4a16_gemm_noalloc_max_bytes(void) { return kScratchBytes; }

int w4a16_gemm_noalloc(const void* packed, int N, int K, int group, int M, const uint16_t* X,
                       int ldx, int had_block, void* Y, int ldy, int y_dtype, void* stream) {
    // every argument, then the size, before the first HIP call
    const int vst = check_gemm_args(packed, N, K, group, M, X, ldx, had_block, Y, ldy, y_dtype);
    if (vst != W4_OK) return vst;
    const size_t need = w4a16_gemm_workspace_bytes(M, K, had_block);
    if (need > kScratchBytes)
        return fail(W4_ERR_SHAPE,
                    "gemm_noalloc: the transform needs %zu bytes, beyond the %zu-byte static "
                    "scratch (M * K * 2 <= %zu)",
                    need, kScratchBytes, kScratchBytes);
    const int dst = check_gemm_disjoint(packed, N, K, group, M, X, ldx, Y, ldy, y_dtype);
    if (dst != W4_OK) return dst;
    void* ws = nullptr;
    if (need) {
        const int st = scratch_ptr(&ws);
        if (st != W4_OK) return st;
    }
    return w4a16_gemm(packed, N, K, group, M, X, ldx, had_block, ws, need ? kScratchBytes : 0, Y,
                      ldy, y_dtype, stream);
}

}  // extern "C"
