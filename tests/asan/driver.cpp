// Host-side memory and undefined-behaviour checks: built with the library's
// host code and the oracle under AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_asan_cpu.py), run on a machine without a GPU.  It exercises
// every path that runs on the host: argument validation of the C ABI (before
// any HIP call), the host packer and unpacker, the dispatcher's tile choice
// and its text, and every oracle routine on small inputs.  Prints ALL OK and
// exits 0; a sanitizer report aborts the run.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "w4a16.h"

extern "C" {
double oracle_bf16_to_f64(uint16_t h);
uint16_t oracle_f64_to_bf16(double v);
int oracle_code(const uint32_t* P, int K, int n, int k);
void oracle_dequant(const uint32_t* P, const uint16_t* S, int N, int K, int group, double* W);
void oracle_gemm(const uint32_t* P, const uint16_t* S, int N, int K, int group,
                 const double* X, int M, int ldx, double* Y, double* A, int nthreads);
void oracle_fwht(const double* X, double* Xout, int M, int K, int block);
void oracle_gather(const uint32_t* P, const uint16_t* S, int N, int K, int group,
                   const int32_t* ids, int B, int out_bf16, void* Y);
void oracle_quantize(const float* W, int N, int K, int ldw, int group, int block,
                     uint32_t* P, uint16_t* S);
void oracle_attn_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V,
                        const int32_t* pos, int H, int T, int D, int cur, int window,
                        double scale, double* out, double* absout);
void oracle_quantize_rows_i8(const float* W, int N, int K, int ldw, int block, int8_t* Q,
                             float* S);
void oracle_gemm_i8(const int8_t* Xq, const float* xs, const int8_t* Wq, const float* ws,
                    int M, int N, int K, double* Y);
}

static int g_fail = 0;

#define CHECK(cond)                                                         \
    do {                                                                    \
        if (!(cond)) {                                                      \
            std::printf("FAIL %s:%d: %s (%s)\n", __FILE__, __LINE__, #cond, \
                        w4_last_error());                                   \
            ++g_fail;                                                       \
        }                                                                   \
    } while (0)

// a fixed-seed 64-bit LCG (Knuth's MMIX constants), top bits
static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd() {
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(g_state >> 32);
}
// a finite bf16 of modest magnitude
static uint16_t rnd_bf16() {
    const uint32_t exp = 120 + rnd() % 12;
    return (uint16_t)(((rnd() & 1) << 15) | (exp << 7) | (rnd() & 0x7F));
}

// Never dereferenced: validation must fail before any access.
static void* const A16 = reinterpret_cast<void*>(0x10000);
static void* const A2 = reinterpret_cast<void*>(0x10002);
static const uint16_t* const X16 = static_cast<const uint16_t*>(A16);

static void validation() {
    // gemv: shape, dtype, NULL and alignment
    CHECK(w4a16_gemv(A16, 256, 512, 64, X16, A16, W4_F32, nullptr) == W4_ERR_SHAPE);
    CHECK(w4a16_gemv(A16, 0, 512, 32, X16, A16, W4_F32, nullptr) == W4_ERR_SHAPE);
    CHECK(w4a16_gemv(A16, 256, 500, 32, X16, A16, W4_F32, nullptr) == W4_ERR_SHAPE);
    CHECK(w4a16_gemv(A16, 256, 512, 32, X16, A16, 7, nullptr) == W4_ERR_DTYPE);
    CHECK(w4a16_gemv(nullptr, 256, 512, 32, X16, A16, W4_F32, nullptr) == W4_ERR_ARG);
    CHECK(w4a16_gemv(A16, 256, 512, 32, nullptr, A16, W4_F32, nullptr) == W4_ERR_ARG);
    CHECK(w4a16_gemv(A2, 256, 512, 32, X16, A16, W4_F32, nullptr) == W4_ERR_ALIGN);
    CHECK(w4a16_gemv(A16, 256, 512, 32, X16, A2, W4_F32, nullptr) == W4_ERR_ALIGN);
    CHECK(w4a16_gemv(A16, 1 << 30, 1 << 20, 32, X16, A16, W4_F32, nullptr) == W4_ERR_SHAPE);
    // small M
    CHECK(w4a16_gemm_smallM(A16, 64, 512, 32, 1, X16, 512, A16, 64, W4_BF16, nullptr) ==
          W4_ERR_SHAPE);
    CHECK(w4a16_gemm_smallM(A16, 64, 512, 32, 4, X16, 516, A16, 64, W4_BF16, nullptr) ==
          W4_ERR_ALIGN);
    // gemm and its allocation-free form
    CHECK(w4a16_gemm(A16, 64, 512, 32, 0, X16, 512, 0, nullptr, 0, A16, 64, W4_BF16,
                     nullptr) == W4_ERR_SHAPE);
    CHECK(w4a16_gemm(A16, 64, 512, 32, 64, X16, 512, 384, nullptr, 0, A16, 64, W4_BF16,
                     nullptr) == W4_ERR_SHAPE);
    CHECK(w4a16_gemm_noalloc(A16, 64, 1 << 20, 256, 1 << 16, X16, 1 << 20, 512, A16, 64,
                             W4_BF16, nullptr) == W4_ERR_SHAPE);
    CHECK(w4a16_gemm_noalloc_max_bytes() > 0);
    // transform
    CHECK(w4_fwht(X16, 512, static_cast<uint16_t*>(A16), 512, 4, 512, 384, nullptr) ==
          W4_ERR_SHAPE);
    // gather, quantize, attention
    CHECK(w4_gather(A16, 64, 512, 48, static_cast<const int32_t*>(A16), 4, A16, 512, W4_BF16,
                    nullptr) == W4_ERR_SHAPE);
    CHECK(w4_gather(A16, 64, 512, 32, nullptr, 4, A16, 512, W4_BF16, nullptr) == W4_ERR_ARG);
    CHECK(w4_gather(A16, 64, 512, 32, nullptr, 0, nullptr, 512, W4_BF16, nullptr) == W4_OK);
    CHECK(w4_quantize(A16, 0, 512, 64, 512, 48, 0, A16, nullptr) == W4_ERR_SHAPE);
    CHECK(w4_quantize(A16, 0, 768, 64, 768, 32, 512, A16, nullptr) == W4_ERR_SHAPE);
    const size_t ws = w4_attn_workspace_bytes(1000, 512);
    CHECK(ws > 0 && w4_attn_workspace_bytes(1000, 384) == 0);
    CHECK(w4_attn_decode(X16, X16, 512, X16, nullptr, 1000, 384, 999, 0, 0.04f, A16, ws, A16,
                         W4_F32, nullptr) == W4_ERR_SHAPE);
    CHECK(w4_attn_decode(X16, X16, 512, X16, nullptr, 1000, 512, 999, 0, NAN, A16, ws, A16,
                         W4_F32, nullptr) == W4_ERR_ARG);
    // sweep creation: bad mode and bad op, before any allocation
    w4_gemv_op op;
    op.packed = A16;
    op.N = 256;
    op.K = 512;
    op.group = 32;
    op.x = X16;
    op.y = A16;
    op.y_dtype = W4_F32;
    w4_sweep* h = nullptr;
    CHECK(w4_decode_sweep_create(&op, 1, 9, nullptr, &h) == W4_ERR_ARG && h == nullptr);
    op.group = 64;
    CHECK(w4_decode_sweep_create(&op, 1, W4_SWEEP_GRAPH, nullptr, &h) == W4_ERR_SHAPE);
    CHECK(w4_decode_sweep_create(nullptr, 1, W4_SWEEP_GRAPH, nullptr, &h) == W4_ERR_ARG);
    CHECK(w4_decode_sweep_destroy(nullptr) == W4_ERR_ARG);
    // status strings
    for (int s = 0; s >= -10; --s) CHECK(std::strcmp(w4_status_str(s), "unknown status") != 0);
    CHECK(std::strcmp(w4_status_str(-1000), "unknown status") == 0);
}

static void packed_sizes() {
    CHECK(w4_packed_bytes(256, 512, 32) == 65536 + 8192);
    CHECK(w4_packed_bytes(1, 32, 32) == 256 + 256);
    CHECK(w4_packed_bytes(0, 512, 32) == 0);
    CHECK(w4_packed_bytes(16, 48, 32) == 0);
    CHECK(w4_packed_bytes(-1, 32, 32) == 0);
    CHECK(w4_packed_bytes(1 << 26, 1 << 20, 32) == 0 || w4_packed_bytes(1 << 26, 1 << 20, 32) > 0);
}

// host packer and unpacker: the documented bijection, on ragged shapes
static void pack_roundtrip() {
    const int shapes[][3] = {{1, 32, 32},    {3, 64, 32},   {17, 512, 256}, {5, 1024, 512},
                             {2, 1536, 32},  {33, 96, 32},  {64, 256, 32},  {7, 8192, 32}};
    for (const auto& sh : shapes) {
        const int N = sh[0], K = sh[1], g = sh[2];
        const size_t bytes = w4_packed_bytes(N, K, g);
        CHECK(bytes > 0);
        std::vector<uint32_t> P((size_t)N * K / 8), P2(P.size());
        std::vector<uint16_t> S((size_t)N * K / g), S2(S.size());
        for (auto& w : P) w = rnd();
        for (auto& s : S) s = rnd_bf16();
        std::vector<uint8_t> packed(bytes, 0xA5);
        CHECK(w4_pack_host(P.data(), S.data(), N, K, g, packed.data()) == W4_OK);
        CHECK(w4_unpack_host(packed.data(), N, K, g, P2.data(), S2.data()) == W4_OK);
        CHECK(P == P2);
        CHECK(S == S2);
        CHECK(w4_pack_host(nullptr, S.data(), N, K, g, packed.data()) == W4_ERR_ARG);
        CHECK(w4_pack_host(P.data(), S.data(), N, K, 48, packed.data()) == W4_ERR_SHAPE);
        CHECK(w4_unpack_host(packed.data(), N, K, g, nullptr, S2.data()) == W4_ERR_ARG);
    }
}

// the dispatcher's choice and its text, over many shapes and short buffers
static void dispatch_text() {
    const int Ms[] = {1, 2, 4, 8, 16, 17, 64, 512};
    const int Ns[] = {1, 31, 256, 1536, 2560, 12288, 262144};
    const int Ks[] = {512, 1536, 2048, 6144, 8192};
    const int gs[] = {32, 256, 512};
    char buf[96];
    for (int M : Ms)
        for (int N : Ns)
            for (int K : Ks)
                for (int g : gs) {
                    const int st = w4_describe_dispatch(M, N, K, g, buf, sizeof buf);
                    CHECK(st == W4_OK || st == W4_ERR_SHAPE);
                    if (st == W4_OK) CHECK(std::strlen(buf) < sizeof buf);
                    char small[6];
                    const int st2 = w4_describe_dispatch(M, N, K, g, small, sizeof small);
                    CHECK(st2 == st);
                    if (st2 == W4_OK) CHECK(std::strlen(small) < sizeof small);
                }
    CHECK(w4_describe_dispatch(1, 256, 512, 32, nullptr, 8) == W4_ERR_ARG);
    CHECK(w4_describe_dispatch(1, 256, 512, 32, buf, 0) == W4_ERR_ARG);
}

static bool finite_all(const double* v, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!std::isfinite(v[i])) return false;
    return true;
}

// every oracle routine on small inputs
static void oracle_routines() {
    const int N = 5, K = 64, g = 32, M = 3;
    std::vector<uint32_t> P((size_t)N * K / 8);
    std::vector<uint16_t> S((size_t)N * K / g);
    for (auto& w : P) w = rnd();
    for (auto& s : S) s = rnd_bf16();
    P[0] = 0x88888888u;   // row 0, codes 0..7: all 8, weight 0
    std::vector<double> W((size_t)N * K);
    oracle_dequant(P.data(), S.data(), N, K, g, W.data());
    for (int k = 0; k < 8; ++k) CHECK(W[k] == 0.0 && oracle_code(P.data(), K, 0, k) == 8);
    CHECK(finite_all(W.data(), W.size()));

    std::vector<double> X((size_t)M * K), Y((size_t)M * N), A((size_t)M * N);
    for (auto& x : X) x = oracle_bf16_to_f64(rnd_bf16());
    oracle_gemm(P.data(), S.data(), N, K, g, X.data(), M, K, Y.data(), A.data(), 1);
    CHECK(finite_all(Y.data(), Y.size()) && finite_all(A.data(), A.size()));
    for (size_t i = 0; i < Y.size(); ++i) CHECK(std::fabs(Y[i]) <= A[i]);

    std::vector<double> Xr(X.size());
    oracle_fwht(X.data(), Xr.data(), M, K, 16);
    CHECK(finite_all(Xr.data(), Xr.size()));

    CHECK(oracle_f64_to_bf16(1.0) == 0x3F80 && oracle_f64_to_bf16(-2.0) == 0xC000);
    CHECK(oracle_bf16_to_f64(oracle_f64_to_bf16(0.15625)) == 0.15625);

    const int32_t ids[4] = {0, 4, -1, 5};   // two out of range: NaN rows
    std::vector<float> G((size_t)4 * K);
    oracle_gather(P.data(), S.data(), N, K, g, ids, 4, 0, G.data());
    for (int k = 0; k < K; ++k)
        CHECK(std::isnan(G[(size_t)2 * K + k]) && std::isnan(G[(size_t)3 * K + k]) &&
              std::isfinite(G[k]));
    std::vector<uint16_t> Gb((size_t)4 * K);
    oracle_gather(P.data(), S.data(), N, K, g, ids, 4, 1, Gb.data());

    std::vector<float> Wf((size_t)N * K);
    for (auto& w : Wf) w = (float)((int)(rnd() % 2001) - 1000) * 1e-3f;
    std::vector<uint32_t> Pq(P.size());
    std::vector<uint16_t> Sq(S.size());
    oracle_quantize(Wf.data(), N, K, K, g, 0, Pq.data(), Sq.data());
    oracle_quantize(Wf.data(), N, K, K, g, 16, Pq.data(), Sq.data());

    const int H = 2, T = 5, D = 8;
    std::vector<uint16_t> q((size_t)H * D), Kc((size_t)T * D), Vc((size_t)T * D);
    for (auto& v : q) v = rnd_bf16();
    for (auto& v : Kc) v = rnd_bf16();
    for (auto& v : Vc) v = rnd_bf16();
    const int32_t pos[5] = {0, 1, 2, 3, 4};
    std::vector<double> o((size_t)H * D), ao((size_t)H * D);
    oracle_attn_decode(q.data(), Kc.data(), Vc.data(), nullptr, H, T, D, T - 1, 0, 0.3, o.data(),
                       ao.data());
    CHECK(finite_all(o.data(), o.size()));
    oracle_attn_decode(q.data(), Kc.data(), Vc.data(), pos, H, T, D, 4, 3, 0.3, o.data(),
                       ao.data());
    CHECK(finite_all(o.data(), o.size()));

    std::vector<int8_t> Q8((size_t)N * K), X8((size_t)M * K);
    std::vector<float> s8(N), xs(M);
    oracle_quantize_rows_i8(Wf.data(), N, K, K, 0, Q8.data(), s8.data());
    oracle_quantize_rows_i8(Wf.data(), M, K, K, 16, X8.data(), xs.data());
    std::vector<double> Y8((size_t)M * N);
    oracle_gemm_i8(X8.data(), xs.data(), Q8.data(), s8.data(), M, N, K, Y8.data());
    CHECK(finite_all(Y8.data(), Y8.size()));
}

int main() {
    validation();
    packed_sizes();
    pack_roundtrip();
    dispatch_text();
    oracle_routines();
    if (g_fail) {
        std::printf("%d check(s) failed\n", g_fail);
        return 1;
    }
    std::printf("ALL OK\n");
    return 0;
}
