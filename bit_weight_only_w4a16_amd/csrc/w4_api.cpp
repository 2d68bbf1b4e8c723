// w4_api.cpp -- the C ABI: validation, dispatch, errors.
//
// Every entry point validates its arguments before its first HIP call, so the
// error paths run on a machine without a GPU.  No HIP call happens when the
// library is loaded.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "w4_config.h"
#include "w4_dispatch.h"

namespace w4 {

static thread_local char g_err[512];

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
}

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

int hip_fail(hipError_t e, const char* what) {
    if (e == hipSuccess) return W4_OK;
    set_error("%s: %s", what, hipGetErrorString(e));
    return W4_ERR_HIP;
}

static bool aligned(const void* p, size_t a) {
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Largest sizes served (indices stay far from overflow).

static int check_weight_shape(int N, int K, int group) {
    if (group != 32 && group != 256 && group != 512)
        return fail(W4_ERR_SHAPE, "group must be 32, 256 or 512 (got %d)", group);
    if (N < 1 || N > kMaxN) return fail(W4_ERR_SHAPE, "N out of range (got %d)", N);
    if (K < group || K > kMaxK || K % group != 0)
        return fail(W4_ERR_SHAPE, "K must be a positive multiple of group %d (got %d)",
                    group, K);
    return W4_OK;
}

static int check_dtype(int ydt) {
    if (ydt != W4_F32 && ydt != W4_BF16)
        return fail(W4_ERR_DTYPE, "output dtype must be W4_F32 or W4_BF16 (got %d)", ydt);
    return W4_OK;
}

static int check_out_ptr(const void* y, int ydt, const char* name) {
    if (!y) return fail(W4_ERR_ARG, "%s is NULL", name);
    if (!aligned(y, ydt == W4_F32 ? 4 : 2))
        return fail(W4_ERR_ALIGN, "%s misaligned for its dtype", name);
    return W4_OK;
}

static int check_in16(const void* p, const char* name) {
    if (!p) return fail(W4_ERR_ARG, "%s is NULL", name);
    if (!aligned(p, 16)) return fail(W4_ERR_ALIGN, "%s must be 16-byte aligned", name);
    return W4_OK;
}

// The output of a product may share no byte with its activations or its
// weights: other workgroups still read them while outputs are written.
static int check_out_disjoint(const void* packed, int N, int K, int group, const void* X,
                              size_t x_bytes, const void* Y, size_t y_bytes, const char* who) {
    if (ranges_overlap(Y, y_bytes, X, x_bytes))
        return fail(W4_ERR_ARG, "%s: the output overlaps the activations", who);
    if (ranges_overlap(Y, y_bytes, packed, w4_packed_bytes(N, K, group)))
        return fail(W4_ERR_ARG, "%s: the output overlaps the weights", who);
    return W4_OK;
}

static size_t rows_bytes(int M, int ld, int n, size_t es) {
    return ((size_t)(M - 1) * (size_t)ld + (size_t)n) * es;
}

}  // namespace w4

using namespace w4;

#define W4_TRY(expr)                 \
    do {                             \
        const int _st = (expr);      \
        if (_st != W4_OK) return _st; \
    } while (0)

namespace w4 {
void log_choice(int M, int N, int K, int group);
}

extern "C" {

const char* w4_status_str(int status) {
    switch (status) {
        case W4_OK: return "ok";
        case W4_ERR_ARG: return "invalid argument";
        case W4_ERR_SHAPE: return "invalid shape";
        case W4_ERR_ALIGN: return "misaligned pointer or stride";
        case W4_ERR_DTYPE: return "invalid dtype";
        case W4_ERR_UNSUPPORTED: return "unsupported";
        case W4_ERR_HIP: return "HIP runtime error";
        case W4_ERR_NOMEM: return "out of memory";
        case W4_ERR_ARCH: return "device is not gfx950";
        case W4_ERR_TIMEOUT: return "in-kernel wait timed out";
        case W4_ERR_SELFTEST: return "self-test output mismatch";
        default: return "unknown status";
    }
}

const char* w4_last_error(void) { return g_err; }

int w4_device_check(void) {
    int dev = 0;
    W4_TRY(hip_fail(hipGetDevice(&dev), "hipGetDevice"));
    hipDeviceProp_t prop;
    W4_TRY(hip_fail(hipGetDeviceProperties(&prop, dev), "hipGetDeviceProperties"));
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(W4_ERR_ARCH, "device %d is %s, this library is built for gfx950",
                    dev, prop.gcnArchName);
    return W4_OK;
}

const char* w4_build_info(void) {
    return "abi=1 arch=gfx950 kernels=gemv,gemv_generic,smallm,fwht,mfma_gemm,sweep_graph,"
           "sweep_persistent,pack,gather,quantize,attn_decode,int8_twin,probe";
}

size_t w4_packed_bytes(int N, int K, int group) {
    if (check_weight_shape(N, K, group) != W4_OK) return 0;
    return packed_bytes(N, K, group);
}

int w4_pack(const uint32_t* P, const uint16_t* S, int N, int K, int group,
            void* out, void* stream) {
    W4_TRY(check_weight_shape(N, K, group));
    if (!P || !S || !out) return fail(W4_ERR_ARG, "w4_pack: NULL pointer");
    if (!aligned(P, 4) || !aligned(S, 2) || !aligned(out, 16))
        return fail(W4_ERR_ALIGN, "w4_pack: P 4-, S 2-, out 16-byte alignment required");
    return launch_pack(P, S, N, K, group, out, static_cast<hipStream_t>(stream));
}

int w4_pack_host(const uint32_t* P, const uint16_t* S, int N, int K, int group,
                 void* out) {
    W4_TRY(check_weight_shape(N, K, group));
    if (!P || !S || !out) return fail(W4_ERR_ARG, "w4_pack_host: NULL pointer");
    uint8_t* base = static_cast<uint8_t*>(out);
    uint32_t* codes = reinterpret_cast<uint32_t*>(base);
    const size_t n_words = (size_t)N * (size_t)(K / 8);
    for (size_t i = 0; i < n_words; ++i) codes[i] = word_to_device(P[i]);
    const size_t off = scale_offset(N, K);
    memset(base + n_words * 4, 0, off - n_words * 4);
    const size_t n_scales = (size_t)N * (size_t)(K / group);
    memcpy(base + off, S, n_scales * 2);
    const size_t total = packed_bytes(N, K, group);
    memset(base + off + n_scales * 2, 0, total - off - n_scales * 2);
    return W4_OK;
}

int w4_unpack_host(const void* packed, int N, int K, int group, uint32_t* P,
                   uint16_t* S) {
    W4_TRY(check_weight_shape(N, K, group));
    if (!packed || !P || !S) return fail(W4_ERR_ARG, "w4_unpack_host: NULL pointer");
    const uint8_t* base = static_cast<const uint8_t*>(packed);
    const uint32_t* codes = reinterpret_cast<const uint32_t*>(base);
    const size_t n_words = (size_t)N * (size_t)(K / 8);
    for (size_t i = 0; i < n_words; ++i) P[i] = word_from_device(codes[i]);
    memcpy(S, base + scale_offset(N, K), (size_t)N * (size_t)(K / group) * 2);
    return W4_OK;
}

int w4a16_gemv(const void* packed, int N, int K, int group, const uint16_t* x,
               void* y, int ydt, void* stream) {
    W4_TRY(check_weight_shape(N, K, group));
    W4_TRY(check_dtype(ydt));
    W4_TRY(check_in16(packed, "packed"));
    W4_TRY(check_in16(x, "x"));
    W4_TRY(check_out_ptr(y, ydt, "y"));
    W4_TRY(config_status());
    const char* src = nullptr;
    const GemvTile t = pick_gemv_tile(N, K, group, &src);
    log_choice(1, N, K, group);
    W4_TRY(check_out_disjoint(packed, N, K, group, x, (size_t)K * 2, y,
                              (size_t)N * (ydt == W4_F32 ? 4 : 2), "gemv"));
    return launch_gemv(t, packed, N, K, group, x, y, ydt,
                       static_cast<hipStream_t>(stream));
}

int w4a16_gemm_smallM(const void* packed, int N, int K, int group, int M,
                      const uint16_t* X, int ldx, void* Y, int ldy, int ydt,
                      void* stream) {
    W4_TRY(check_weight_shape(N, K, group));
    W4_TRY(check_dtype(ydt));
    if (M < 2 || M > 16) return fail(W4_ERR_SHAPE, "smallM: M must be in 2..16 (got %d)", M);
    if (ldx < K || ldy < N) return fail(W4_ERR_SHAPE, "smallM: ldx >= K and ldy >= N required");
    if (ldx % 8 != 0) return fail(W4_ERR_ALIGN, "smallM: ldx must be a multiple of 8");
    W4_TRY(check_in16(packed, "packed"));
    W4_TRY(check_in16(X, "X"));
    W4_TRY(check_out_ptr(Y, ydt, "Y"));
    W4_TRY(config_status());
    log_choice(M, N, K, group);
    W4_TRY(check_out_disjoint(packed, N, K, group, X, rows_bytes(M, ldx, K, 2), Y,
                              rows_bytes(M, ldy, N, ydt == W4_F32 ? 4 : 2), "smallM"));
    return launch_smallm(packed, N, K, group, M, X, ldx, Y, ldy, ydt,
                         static_cast<hipStream_t>(stream));
}

int w4_fwht(const uint16_t* X, int ldx, uint16_t* Xo, int ldo, int M, int K,
            int block, void* stream) {
    if (block < 2 || block > 1024 || (block & (block - 1)) != 0)
        return fail(W4_ERR_SHAPE, "fwht: block must be a power of two in 2..1024 (got %d)", block);
    if (M < 1 || K < block || K % block != 0 || K > kMaxK)
        return fail(W4_ERR_SHAPE, "fwht: K must be a positive multiple of block");
    if (ldx < K || ldo < K) return fail(W4_ERR_SHAPE, "fwht: ldx, ldo >= K required");
    if (ldx % 8 != 0 || ldo % 8 != 0)
        return fail(W4_ERR_ALIGN, "fwht: ldx and ldo must be multiples of 8");
    W4_TRY(check_in16(X, "X"));
    W4_TRY(check_in16(Xo, "Xout"));
    if (X == Xo && ldx != ldo) return fail(W4_ERR_ARG, "fwht: in place needs ldo == ldx");
    return launch_fwht(X, ldx, Xo, ldo, M, K, block, static_cast<hipStream_t>(stream));
}

// w4a16_gemm: largest row count that always takes the small-M product
constexpr int kGemmSmallMRows = 8;
// w4a16_gemm: largest row count whose transform runs inside the small-M kernel
constexpr int kGemmFusedTransformRows = 4;

size_t w4a16_gemm_workspace_bytes(int M, int K, int had_block) {
    if (had_block == 0 || M < 1 || K < 1) return 0;
    return align_up((size_t)M * (size_t)K * 2, kAlign);
}

}  // extern "C"

namespace w4 {

int check_gemm_args(const void* packed, int N, int K, int group, int M, const uint16_t* X,
                    int ldx, int had_block, const void* Y, int ldy, int ydt) {
    W4_TRY(check_weight_shape(N, K, group));
    W4_TRY(check_dtype(ydt));
    if (M < 1 || M > (1 << 20)) return fail(W4_ERR_SHAPE, "gemm: M out of range (got %d)", M);
    if (K % 256 != 0) return fail(W4_ERR_SHAPE, "gemm: K must be a multiple of 256");
    if (ldx < K || ldy < N) return fail(W4_ERR_SHAPE, "gemm: ldx >= K and ldy >= N required");
    if (ldx % 8 != 0) return fail(W4_ERR_ALIGN, "gemm: ldx must be a multiple of 8");
    if (had_block != 0 &&
        (had_block < 2 || had_block > 1024 || (had_block & (had_block - 1)) != 0 ||
         K % had_block != 0))
        return fail(W4_ERR_SHAPE, "gemm: had_block must be 0 or a power of two dividing K");
    W4_TRY(check_in16(packed, "packed"));
    W4_TRY(check_in16(X, "X"));
    W4_TRY(check_out_ptr(Y, ydt, "Y"));
    return W4_OK;
}

int check_gemm_disjoint(const void* packed, int N, int K, int group, int M, const uint16_t* X,
                        int ldx, const void* Y, int ldy, int ydt) {
    return check_out_disjoint(packed, N, K, group, X, rows_bytes(M, ldx, K, 2), Y,
                              rows_bytes(M, ldy, N, ydt == W4_F32 ? 4 : 2), "gemm");
}

// W4_LOG: the kernel and tile each distinct (M, N, K, group) dispatches to,
// printed once.
void log_choice(int M, int N, int K, int group) {
    const auto c = config();
    if (!c->log) return;
    char d[192];
    if (w4_describe_dispatch(M, N, K, group, d, sizeof d) != W4_OK) return;
    char line[256];
    snprintf(line, sizeof line, "M=%d N=%d K=%d group=%d: %s", M, N, K, group, d);
    log_dispatch(*c, line);
}

}  // namespace w4

extern "C" {

int w4_config_reload(void) { return reload_config(); }

int w4_tile_table_load(const char* path) { return load_tile_table(path); }


int w4a16_gemm(const void* packed, int N, int K, int group, int M,
               const uint16_t* X, int ldx, int had_block, void* workspace,
               size_t ws_bytes, void* Y, int ldy, int ydt, void* stream) {
    W4_TRY(check_gemm_args(packed, N, K, group, M, X, ldx, had_block, Y, ldy, ydt));
    W4_TRY(config_status());
    log_choice(M, N, K, group);
    const size_t need = w4a16_gemm_workspace_bytes(M, K, had_block);
    if (need) {
        if (ws_bytes < need)
            return fail(W4_ERR_SHAPE, "gemm: workspace of %zu bytes needed (got %zu)", need,
                        ws_bytes);
        W4_TRY(check_in16(workspace, "workspace"));
    }
    W4_TRY(check_gemm_disjoint(packed, N, K, group, M, X, ldx, Y, ldy, ydt));
    hipStream_t s = static_cast<hipStream_t>(stream);
    // The 512-block transform of up to 4 rows runs inside the matrix-core
    // small-M kernel, on the rows it stages anyway (bitwise the same rows the
    // transform kernel writes; the workspace goes unused).  Every workgroup
    // transforms all rows itself, so from 8 rows on the separate transform
    // kernel is faster (measured at N = 12288, K = 1536: fused 6.7 / 7.9 /
    // 9.8 us at 2 / 4 / 8 rows, separate 8.1 / 8.3 / 8.7 us).
    if (had_block == 512 && M >= 2 && M <= kGemmFusedTransformRows &&
        smallm_mfma_applies(M, N, K, group))
        return launch_smallm(packed, N, K, group, M, X, ldx, Y, ldy, ydt, s, 512);
    const uint16_t* Xin = X;
    int ld_in = ldx;
    if (had_block) {
        uint16_t* Xr = static_cast<uint16_t*>(workspace);
        W4_TRY(launch_fwht(X, ldx, Xr, K, M, K, had_block, s));
        Xin = Xr;
        ld_in = K;
    }
    // Few rows are decode-shaped ([P2] "fastgemma"): the small-M product,
    // which for the rotated formats (groups 256 and 512) multiplies one
    // 16-row tile on the matrix cores and is then the fastest through 16 rows
    // (measured at N = 12288, K = 1536: 5.6 us at 8 rows, 6.3 us at 16,
    // against 11.3 us on the tiled matrix-core kernel); otherwise the
    // vector-ALU small-M kernel up to 8 rows (10.1 us at 8, 18..25 us at
    // 9..16) and the tiled kernel from 9 rows.
    if (M == 1) {
        const GemvTile t = pick_gemv_tile(N, K, group);
        return launch_gemv(t, packed, N, K, group, Xin, Y, ydt, s);
    }
    if (splitk_applies(M, N, K, group, ld_in))
        return launch_splitk(packed, N, K, group, M, Xin, ld_in, Y, ldy, ydt, s);
    if (M <= kGemmSmallMRows || (M <= 16 && smallm_mfma_applies(M, N, K, group)))
        return launch_smallm(packed, N, K, group, M, Xin, ld_in, Y, ldy, ydt, s);
    return launch_mfma_gemm(packed, N, K, group, M, Xin, ld_in, Y, ldy, ydt, s);
}

int w4_gather(const void* packed, int N, int K, int group, const int32_t* ids, int B,
              void* Y, int ldy, int ydt, void* stream) {
    W4_TRY(check_weight_shape(N, K, group));
    W4_TRY(check_in16(packed, "packed"));
    W4_TRY(check_dtype(ydt));
    if (B < 0 || B > (1 << 24)) return fail(W4_ERR_SHAPE, "gather: B out of range (got %d)", B);
    if (B == 0) return W4_OK;
    if (!ids) return fail(W4_ERR_ARG, "gather: ids is NULL");
    if (!aligned(ids, 4)) return fail(W4_ERR_ALIGN, "gather: ids must be 4-byte aligned");
    W4_TRY(check_in16(Y, "Y"));
    if (ldy < K) return fail(W4_ERR_SHAPE, "gather: ldy %d < K %d", ldy, K);
    if (ldy % (ydt == W4_F32 ? 4 : 8) != 0)
        return fail(W4_ERR_ALIGN, "gather: rows of Y must start 16-byte aligned (ldy %d)", ldy);
    return launch_gather(packed, N, K, group, ids, B, Y, ldy, ydt,
                         static_cast<hipStream_t>(stream));
}

int w4_quantize(const void* W, int w_dtype, int ldw, int N, int K, int group, int had_block,
                void* packed, void* stream) {
    W4_TRY(check_weight_shape(N, K, group));
    if (w_dtype != W4_F32 && w_dtype != W4_BF16)
        return fail(W4_ERR_DTYPE, "quantize: W dtype must be W4_F32 or W4_BF16 (got %d)", w_dtype);
    if (had_block != 0 && had_block != 64 && had_block != 128 && had_block != 256 &&
        had_block != 512)
        return fail(W4_ERR_SHAPE, "quantize: had_block must be 0, 64, 128, 256 or 512 (got %d)",
                    had_block);
    if (had_block && K % had_block != 0)
        return fail(W4_ERR_SHAPE, "quantize: K %d not a multiple of had_block %d", K, had_block);
    W4_TRY(check_in16(W, "W"));
    W4_TRY(check_in16(packed, "packed"));
    if (ldw < K) return fail(W4_ERR_SHAPE, "quantize: ldw %d < K %d", ldw, K);
    if (ldw % (w_dtype == W4_F32 ? 4 : 8) != 0)
        return fail(W4_ERR_ALIGN, "quantize: rows of W must start 16-byte aligned (ldw %d)", ldw);
    return launch_quantize(W, w_dtype, ldw, N, K, group, had_block, packed,
                           static_cast<hipStream_t>(stream));
}

static int check_had_block(int K, int had_block, const char* what) {
    if (had_block != 0 && had_block != 64 && had_block != 128 && had_block != 256 &&
        had_block != 512)
        return fail(W4_ERR_SHAPE, "%s: had_block must be 0, 64, 128, 256 or 512 (got %d)", what,
                    had_block);
    if (had_block && K % had_block != 0)
        return fail(W4_ERR_SHAPE, "%s: K %d not a multiple of had_block %d", what, K, had_block);
    return W4_OK;
}

int w4_quantize_rows_i8(const void* X, int x_dtype, int ldx, int N, int K, int had_block,
                        int8_t* Q, int ldq, float* S, void* stream) {
    if (x_dtype != W4_F32 && x_dtype != W4_BF16)
        return fail(W4_ERR_DTYPE, "int8 quantize: dtype must be W4_F32 or W4_BF16 (got %d)",
                    x_dtype);
    if (N < 1 || N > kMaxN) return fail(W4_ERR_SHAPE, "int8 quantize: N out of range (got %d)", N);
    if (K < 8 || K > kMaxK || K % 8 != 0)
        return fail(W4_ERR_SHAPE, "int8 quantize: K must be a positive multiple of 8 (got %d)", K);
    W4_TRY(check_had_block(K, had_block, "int8 quantize"));
    W4_TRY(check_in16(X, "X"));
    W4_TRY(check_in16(Q, "Q"));
    if (!S) return fail(W4_ERR_ARG, "int8 quantize: S is NULL");
    if (!aligned(S, 4)) return fail(W4_ERR_ALIGN, "int8 quantize: S must be 4-byte aligned");
    if (ldx < K || ldx % (x_dtype == W4_F32 ? 4 : 8) != 0)
        return fail(W4_ERR_ALIGN, "int8 quantize: ldx must be >= K with 16-byte aligned rows");
    if (ldq < K || ldq % 8 != 0)
        return fail(W4_ERR_ALIGN, "int8 quantize: ldq must be >= K and a multiple of 8");
    return launch_quantize_rows_i8(X, x_dtype, ldx, N, K, had_block, Q, ldq, S,
                                   static_cast<hipStream_t>(stream));
}

int w4_gemm_i8(const int8_t* Xq, int ldx, const float* xs, const int8_t* Wq, int ldw,
               const float* ws, int M, int N, int K, void* Y, int ldy, int ydt, void* stream) {
    if (M < 1 || M > kMaxN || N < 1 || N > kMaxN)
        return fail(W4_ERR_SHAPE, "int8 gemm: M or N out of range (%d, %d)", M, N);
    if (K < 128 || K > kMaxK || K % 128 != 0)
        return fail(W4_ERR_SHAPE, "int8 gemm: K must be a positive multiple of 128 (got %d)", K);
    W4_TRY(check_dtype(ydt));
    W4_TRY(check_in16(Xq, "Xq"));
    W4_TRY(check_in16(Wq, "Wq"));
    if (!xs || !ws) return fail(W4_ERR_ARG, "int8 gemm: scales NULL");
    if (!aligned(xs, 4) || !aligned(ws, 4))
        return fail(W4_ERR_ALIGN, "int8 gemm: scales must be 4-byte aligned");
    if (ldx < K || ldx % 16 != 0 || ldw < K || ldw % 16 != 0)
        return fail(W4_ERR_ALIGN, "int8 gemm: ldx and ldw must be >= K and multiples of 16");
    W4_TRY(check_out_ptr(Y, ydt, "Y"));
    if (ldy < N) return fail(W4_ERR_SHAPE, "int8 gemm: ldy %d < N %d", ldy, N);
    W4_TRY(config_status());
    if (config()->log) {
        char d[128], line[200];
        describe_i8(M, N, K, d, sizeof d);
        snprintf(line, sizeof line, "int8 M=%d N=%d K=%d: %s", M, N, K, d);
        log_dispatch(*config(), line);
    }
    return launch_gemm_i8(Xq, ldx, xs, Wq, ldw, ws, M, N, K, Y, ldy, ydt,
                          static_cast<hipStream_t>(stream));
}

size_t w4a16_gemm_twin_workspace_bytes(int M, int K, int had_block, int switch_rows) {
    if (M < 1 || K < 1) return 0;
    if (M < switch_rows) return w4a16_gemm_workspace_bytes(M, K, had_block);
    return align_up((size_t)M * (size_t)K, kAlign) + (size_t)M * sizeof(float);
}

int w4a16_gemm_twin(const void* packed4, const int8_t* W8, int ldw8, const float* ws8, int N,
                    int K, int group, int M, const uint16_t* X, int ldx, int had_block,
                    int switch_rows, void* workspace, size_t ws_bytes, void* Y, int ldy, int ydt,
                    void* stream) {
    if (switch_rows < 1) return fail(W4_ERR_ARG, "twin: switch_rows must be >= 1");
    if (M < switch_rows)
        return w4a16_gemm(packed4, N, K, group, M, X, ldx, had_block, workspace, ws_bytes, Y, ldy,
                          ydt, stream);
    W4_TRY(check_weight_shape(N, K, group));
    W4_TRY(check_had_block(K, had_block, "twin"));
    if (K % 128 != 0) return fail(W4_ERR_SHAPE, "twin: K must be a multiple of 128 (got %d)", K);
    const size_t need = w4a16_gemm_twin_workspace_bytes(M, K, had_block, switch_rows);
    W4_TRY(check_in16(workspace, "workspace"));
    if (ws_bytes < need)
        return fail(W4_ERR_SHAPE, "twin: workspace %zu bytes < %zu", ws_bytes, need);
    if (!W8 || !ws8) return fail(W4_ERR_ARG, "twin: int8 twin NULL");
    int8_t* Xq = static_cast<int8_t*>(workspace);
    float* xs = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                         align_up((size_t)M * (size_t)K, kAlign));
    // validate the product's arguments before the first launch
    if (ldw8 < K || ldw8 % 16 != 0 || !aligned(W8, 16) || !aligned(ws8, 4))
        return fail(W4_ERR_ALIGN, "twin: W8 rows must be 16-byte aligned (ldw8 >= K, %% 16)");
    W4_TRY(check_dtype(ydt));
    W4_TRY(check_out_ptr(Y, ydt, "Y"));
    if (ldy < N) return fail(W4_ERR_SHAPE, "twin: ldy %d < N %d", ldy, N);
    W4_TRY(w4_quantize_rows_i8(X, W4_BF16, ldx, M, K, had_block, Xq, K, xs, stream));
    return w4_gemm_i8(Xq, K, xs, W8, ldw8, ws8, M, N, K, Y, ldy, ydt, stream);
}

static int check_attn_shape(int T, int D) {
    if (D != 256 && D != 512) return fail(W4_ERR_SHAPE, "attention: D must be 256 or 512 (got %d)", D);
    if (T < 1 || T > (1 << 24)) return fail(W4_ERR_SHAPE, "attention: T out of range (got %d)", T);
    return W4_OK;
}

size_t w4_attn_workspace_bytes(int T, int D) {
    if (check_attn_shape(T, D) != W4_OK) return 0;
    return attn_workspace_bytes(T, D);
}

int w4_attn_decode(const uint16_t* q, const uint16_t* K, int ldk, const uint16_t* Vt,
                   const int32_t* pos, int T, int D, int cur, int window, float scale,
                   void* workspace, size_t ws_bytes, void* out, int out_dtype, void* stream) {
    W4_TRY(check_attn_shape(T, D));
    W4_TRY(check_dtype(out_dtype));
    W4_TRY(check_in16(q, "q"));
    W4_TRY(check_in16(K, "K"));
    W4_TRY(check_in16(Vt, "Vt"));
    W4_TRY(check_in16(workspace, "workspace"));
    W4_TRY(check_in16(out, "out"));
    if (ldk < D || ldk % 8 != 0)
        return fail(W4_ERR_ALIGN, "attention: ldk must be >= D and a multiple of 8 (got %d)", ldk);
    if (pos && !aligned(pos, 4)) return fail(W4_ERR_ALIGN, "attention: pos must be 4-byte aligned");
    if (window < 0) return fail(W4_ERR_ARG, "attention: window < 0");
    if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f)
        return fail(W4_ERR_ARG, "attention: scale must be finite");
    if (ws_bytes < attn_workspace_bytes(T, D))
        return fail(W4_ERR_SHAPE, "attention: workspace %zu bytes < %zu", ws_bytes,
                    attn_workspace_bytes(T, D));
    return launch_attn_decode(q, K, ldk, Vt, pos, T, D, cur, window, scale, workspace, out,
                              out_dtype, static_cast<hipStream_t>(stream));
}

int w4_attn_pack_v(const uint16_t* V, int ldv, int T, int D, uint16_t* Vt, void* stream) {
    W4_TRY(check_attn_shape(T, D));
    if (!V) return fail(W4_ERR_ARG, "attention: V is NULL");
    if (!aligned(V, 2)) return fail(W4_ERR_ALIGN, "attention: V must be 2-byte aligned");
    W4_TRY(check_in16(Vt, "Vt"));
    if (ldv < D) return fail(W4_ERR_SHAPE, "attention: ldv %d < D %d", ldv, D);
    return launch_attn_pack_v(V, ldv, T, D, Vt, static_cast<hipStream_t>(stream));
}

int w4_attn_store_kv(const uint16_t* k, const uint16_t* v, int slot, uint16_t* K, int ldk,
                     uint16_t* Vt, int D, void* stream) {
    W4_TRY(check_attn_shape(1, D));
    if (!k || !v || !K || !Vt) return fail(W4_ERR_ARG, "attention: NULL pointer");
    if (!aligned(k, 2) || !aligned(v, 2) || !aligned(K, 2) || !aligned(Vt, 2))
        return fail(W4_ERR_ALIGN, "attention: pointers must be 2-byte aligned");
    if (slot < 0 || slot >= (1 << 24)) return fail(W4_ERR_SHAPE, "attention: slot out of range");
    if (ldk < D) return fail(W4_ERR_SHAPE, "attention: ldk %d < D %d", ldk, D);
    return launch_attn_store_kv(k, v, slot, K, ldk, Vt, D, static_cast<hipStream_t>(stream));
}

int w4_describe_dispatch(int M, int N, int K, int group, char* buf, size_t len) {
    W4_TRY(check_weight_shape(N, K, group));
    if (!buf || len == 0) return fail(W4_ERR_ARG, "describe: empty buffer");
    if (M < 1) return fail(W4_ERR_SHAPE, "describe: M must be >= 1");
    W4_TRY(config_status());
    if (M == 1) {
        const char* src = nullptr;
        const GemvTile t = pick_gemv_tile(N, K, group, &src);
        snprintf(buf, len, "gemv%s L=%d U=%d W=%d grid=%d stages=%d%s (%s)",
                 t.generic ? "_generic" : "", t.L, t.U, t.waves, t.grid, t.stages,
                 t.contig ? " contiguous" : "", src);
    } else if (splitk_applies(M, N, K, group, K)) {
        describe_splitk(M, N, K, group, K, buf, len);
  } else if (M <= kGemmSmallMRows || (M <= 16 && smallm_mfma_applies(M, N, K, group))) {
        describe_smallm(M, N, K, group, buf, len);
    } else {
        if (K % 256 != 0) return fail(W4_ERR_SHAPE, "describe: gemm needs K % 256 == 0");
        describe_mfma(M, N, K, group, buf, len);
    }
    return W4_OK;
}

int w4_probe_read(const void* buf, size_t bytes, uint32_t* out, void* stream) {
    W4_TRY(check_in16(buf, "buf"));
    if (!out) return fail(W4_ERR_ARG, "probe: out is NULL");
    if (!aligned(out, 4)) return fail(W4_ERR_ALIGN, "probe: out must be 4-byte aligned");
    if (bytes == 0 || bytes % 16 != 0)
        return fail(W4_ERR_SHAPE, "probe: bytes must be a positive multiple of 16");
    return launch_probe_read(buf, bytes, out, static_cast<hipStream_t>(stream));
}

int w4_probe_mfma(int iters, float* out, void* stream) {
    if (iters < 1 || iters > (1 << 20))
        return fail(W4_ERR_SHAPE, "probe: iters must be in 1..2^20 (got %d)", iters);
    if (!out) return fail(W4_ERR_ARG, "probe: out is NULL");
    if (!aligned(out, 4)) return fail(W4_ERR_ALIGN, "probe: out must be 4-byte aligned");
    return launch_probe_mfma(iters, out, static_cast<hipStream_t>(stream));
}

size_t w4_probe_handoff_bytes(void) { return probe_handoff_bytes(); }

int w4_probe_handoff(void* work, int rounds, int rows, void* stream) {
    if (!work) return fail(W4_ERR_ARG, "probe handoff: work is NULL");
    if (!aligned(work, 256)) return fail(W4_ERR_ALIGN, "probe handoff: work must be 256-byte aligned");
    if (rounds < 1 || rounds > (1 << 20))
        return fail(W4_ERR_SHAPE, "probe handoff: rounds must be in 1..2^20 (got %d)", rounds);
    if (rows < 0 || rows > 64)
        return fail(W4_ERR_SHAPE, "probe handoff: rows must be in 0..64 (got %d)", rows);
    return launch_probe_handoff(work, rounds, rows, static_cast<hipStream_t>(stream));
}

int w4_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
    W4_TRY(check_in16(src, "src"));
    W4_TRY(check_in16(dst, "dst"));
    if (bytes == 0 || bytes % 16 != 0)
        return fail(W4_ERR_SHAPE, "probe: bytes must be a positive multiple of 16");
    return launch_probe_copy(src, dst, bytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"
