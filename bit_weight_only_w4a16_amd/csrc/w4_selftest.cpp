// w4_selftest.cpp -- start-up check of the compute paths on the current GPU.
//
// [P2] "fastgemma -- Gemma 4 E2B, CPU-only, AMX INT8 / AVX-512 VNNI" probes
// its machine at start-up before trusting a kernel path.  Here every product
// path runs on small built-in matrices with one-hot activations: a one-hot x
// (a single bf16 1.0 at column k) makes output n exactly (code(n,k) - 8) *
// scale(n, k / group), a small integer times a bf16, which fp32 holds
// exactly.  So the expected outputs are known in closed form and the check is
// bitwise.  Covered: the batch-1 GEMV (group 32 and 256), the small-M kernel
// (M = 8) and the matrix-core GEMM (M = 64), each through the public entry
// points, so dispatch is exercised as callers see it.
#include <cstring>
#include <vector>

#include "w4_dispatch.h"

extern "C" {
int w4_device_check(void);
int w4_pack(const uint32_t* P, const uint16_t* S, int N, int K, int group, void* out,
            void* stream);
size_t w4_packed_bytes(int N, int K, int group);
int w4a16_gemv(const void* packed, int N, int K, int group, const uint16_t* x, void* y,
               int ydt, void* stream);
int w4a16_gemm_smallM(const void* packed, int N, int K, int group, int M, const uint16_t* X,
                      int ldx, void* Y, int ldy, int ydt, void* stream);
int w4a16_gemm(const void* packed, int N, int K, int group, int M, const uint16_t* X, int ldx,
               int had_block, void* workspace, size_t ws_bytes, void* Y, int ldy, int ydt,
               void* stream);
}

namespace w4 {
namespace {

constexpr int kN = 100;  // rows: not a multiple of any tile height
constexpr int kK = 512;
constexpr int kM = 64;
constexpr uint16_t kScales[4] = {0x3F80, 0x3FC0, 0x3E80, 0x4040};  // 1, 1.5, 0.25, 3

int code_at(int n, int k) { return (3 * n + 5 * k + (k >> 3)) & 15; }
uint16_t scale_at(int n, int g) { return kScales[(n + g) & 3]; }
int onehot_col(int m) { return (m * 37 + 11) % kK; }

float bf16_value(uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

struct DeviceBuffers {
    std::vector<void*> ptrs;
    void* get(size_t bytes) {
        void* p = nullptr;
        if (hipMalloc(&p, bytes) != hipSuccess) return nullptr;
        ptrs.push_back(p);
        return p;
    }
    ~DeviceBuffers() {
        for (void* p : ptrs) (void)hipFree(p);
    }
};

// Runs one group size through every path; returns a status.
int check_group(int group, hipStream_t s, DeviceBuffers& mem) {
    const int G = kK / group;
    std::vector<uint32_t> P((size_t)kN * (kK / 8), 0u);
    std::vector<uint16_t> S((size_t)kN * G);
    for (int n = 0; n < kN; ++n) {
        for (int k = 0; k < kK; ++k)
            P[(size_t)n * (kK / 8) + k / 8] |= (uint32_t)code_at(n, k) << (4 * (k % 8));
        for (int g = 0; g < G; ++g) S[(size_t)n * G + g] = scale_at(n, g);
    }
    std::vector<uint16_t> X((size_t)kM * kK, 0);
    for (int m = 0; m < kM; ++m) X[(size_t)m * kK + onehot_col(m)] = 0x3F80;

    const size_t pb = w4_packed_bytes(kN, kK, group);
    void* dP = mem.get(P.size() * 4);
    void* dS = mem.get(S.size() * 2);
    void* dW = mem.get(pb);
    void* dX = mem.get(X.size() * 2);
    void* dY = mem.get((size_t)kM * kN * 4);
    if (!dP || !dS || !dW || !dX || !dY) return fail(W4_ERR_NOMEM, "selftest: device allocation");
    int st = hip_fail(hipMemcpyAsync(dP, P.data(), P.size() * 4, hipMemcpyHostToDevice, s),
                      "selftest upload");
    if (st == W4_OK)
        st = hip_fail(hipMemcpyAsync(dS, S.data(), S.size() * 2, hipMemcpyHostToDevice, s),
                      "selftest upload");
    if (st == W4_OK)
        st = hip_fail(hipMemcpyAsync(dX, X.data(), X.size() * 2, hipMemcpyHostToDevice, s),
                      "selftest upload");
    if (st == W4_OK)
        st = w4_pack(static_cast<const uint32_t*>(dP), static_cast<const uint16_t*>(dS), kN, kK,
                     group, dW, s);
    if (st != W4_OK) return st;

    struct Path { const char* name; int M; };
    const Path paths[3] = {{"gemv", 1}, {"smallM", 8}, {"matrix-core gemm", kM}};
    std::vector<float> Y((size_t)kM * kN);
    const uint16_t* x = static_cast<const uint16_t*>(dX);
    for (const Path& p : paths) {
        st = hip_fail(hipMemsetAsync(dY, 0xFF, (size_t)kM * kN * 4, s), "selftest clear");
        if (st != W4_OK) return st;
        if (p.M == 1)
            st = w4a16_gemv(dW, kN, kK, group, x, dY, W4_F32, s);
        else if (p.M <= 16)
            st = w4a16_gemm_smallM(dW, kN, kK, group, p.M, x, kK, dY, kN, W4_F32, s);
        else
            st = w4a16_gemm(dW, kN, kK, group, p.M, x, kK, 0, nullptr, 0, dY, kN, W4_F32, s);
        if (st != W4_OK) return st;
        st = hip_fail(hipMemcpyAsync(Y.data(), dY, (size_t)p.M * kN * 4, hipMemcpyDeviceToHost,
                                     s), "selftest download");
        if (st == W4_OK) st = hip_fail(hipStreamSynchronize(s), "selftest sync");
        if (st != W4_OK) return st;
        for (int m = 0; m < p.M; ++m) {
            const int k = onehot_col(m);
            for (int n = 0; n < kN; ++n) {
                const float want = (float)(code_at(n, k) - 8) * bf16_value(scale_at(n, k / group));
                const float got = Y[(size_t)m * kN + n];
                if (std::memcmp(&want, &got, 4) != 0)
                    return fail(W4_ERR_SELFTEST,
                                "selftest: %s (group %d) row %d output %d: got %.9g, want %.9g",
                                p.name, group, m, n, (double)got, (double)want);
            }
        }
    }
    return W4_OK;
}

}  // namespace
}  // namespace w4

using namespace w4;

extern "C" int w4_selftest(void* stream) {
    int st = w4_device_check();
    if (st != W4_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    DeviceBuffers mem;
    st = check_group(32, s, mem);
    if (st == W4_OK) st = check_group(256, s, mem);
    // buffers are freed only after the stream has drained
    const int sync = hip_fail(hipStreamSynchronize(s), "selftest sync");
    return st != W4_OK ? st : sync;
}
