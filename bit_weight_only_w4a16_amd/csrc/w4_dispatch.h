// w4_dispatch.h -- tile selection and kernel launchers (internal).
#pragma once

#include "w4_common.h"

namespace w4 {

constexpr int kNumCUs = 256;        // MI355X: 8 XCDs x 32 CUs
constexpr int kMaxU = 8;            // 32-element chunks held per lane
constexpr int kMaxN = 1 << 26;      // largest N the entry points accept
constexpr int kMaxK = 1 << 20;      // largest K

// Batch-1 GEMV tiling: L lanes share one row (each lane owns U chunks of K,
// chunk index lane + L*u), a wave covers 64/L rows per step, `waves` waves per
// workgroup, `grid` workgroups; generic = chunks re-read per row (huge K).
struct GemvTile {
    int L = 16;
    int U = 3;
    int waves = 4;
    int grid = 1;          // workgroups (0 in a table entry: chosen from the shape)
    int stages = 2;        // row groups in flight + 1 (2 or 3; 3 for U <= 4)
    bool generic = false;
    bool contig = false;   // contiguous row-group ranges per wave (large N)
};

// The tile for a batch-1 GEMV: W4_FORCE_PATH, then the loaded tile table,
// then the built-in table, then the heuristic; *source (if given) names which.
GemvTile pick_gemv_tile(int N, int K, int group, const char** source = nullptr);

// True when the byte ranges [a, a + na) and [b, b + nb) share a byte.
inline bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

// Argument validation of w4a16_gemm (no HIP call); W4_OK or a status.
int check_gemm_args(const void* packed, int N, int K, int group, int M, const uint16_t* X,
                    int ldx, int had_block, const void* Y, int ldy, int ydt);
// The output span of w4a16_gemm shares no byte with X's span or the weights.
int check_gemm_disjoint(const void* packed, int N, int K, int group, int M, const uint16_t* X,
                        int ldx, const void* Y, int ldy, int ydt);
int launch_gemv(const GemvTile& t, const void* packed, int N, int K, int group,
                const uint16_t* x, void* y, int ydt, hipStream_t s);

int launch_pack(const uint32_t* P, const uint16_t* S, int N, int K, int group,
                void* out, hipStream_t s);

// had_block: 0, or 512 to apply the blockwise transform to X inside the
// matrix-core small-M kernel (only where smallm_mfma_applies)
int launch_smallm(const void* packed, int N, int K, int group, int M,
                  const uint16_t* X, int ldx, void* Y, int ldy, int ydt,
                  hipStream_t s, int had_block = 0);
void describe_smallm(int M, int N, int K, int group, char* buf, size_t len);
// the matrix-core small-M kernel takes this shape (rotated groups, M <= 16)
bool smallm_mfma_applies(int M, int N, int K, int group);

// The split-K matrix-core kernel for 2..64 rows (w4_splitk.hip).
bool splitk_applies(int M, int N, int K, int group, int ldx);
int launch_splitk(const void* packed, int N, int K, int group, int M, const uint16_t* X, int ldx,
                  void* Y, int ldy, int ydt, hipStream_t s);
void describe_splitk(int M, int N, int K, int group, int ldx, char* buf, size_t len);

int launch_fwht(const uint16_t* X, int ldx, uint16_t* Xo, int ldo, int M,
                int K, int block, hipStream_t s);

int launch_mfma_gemm(const void* packed, int N, int K, int group, int M,
                     const uint16_t* X, int ldx, void* Y, int ldy, int ydt,
                     hipStream_t s);
void describe_mfma(int M, int N, int K, int group, char* buf, size_t len);

// DMA-ring prefill kernel (w4_prefill.hip): groups that are multiples of 64
bool prefill_supported(int M, int N, int K, int group, int ldx);
int launch_prefill(const void* packed, int N, int K, int group, int M, const uint16_t* X,
                   int ldx, void* Y, int ldy, int ydt, hipStream_t s);
void describe_prefill(int M, int N, int K, int group, char* buf, size_t len);

int launch_gather(const void* packed, int N, int K, int group, const int32_t* ids, int B,
                  void* Y, int ldy, int ydt, hipStream_t s);

int launch_quantize(const void* W, int wdt, int ldw, int N, int K, int group, int block,
                    void* packed, hipStream_t s);

size_t attn_workspace_bytes(int T, int D);
int launch_attn_decode(const uint16_t* q, const uint16_t* K, int ldk, const uint16_t* Vt,
                       const int32_t* pos, int T, int D, int cur, int window, float scale,
                       void* ws, void* out, int odt, hipStream_t s);
int launch_attn_pack_v(const uint16_t* V, int ldv, int T, int D, uint16_t* Vt, hipStream_t s);
int launch_attn_store_kv(const uint16_t* k, const uint16_t* v, int slot, uint16_t* K, int ldk,
                         uint16_t* Vt, int D, hipStream_t s);

int launch_quantize_rows_i8(const void* W, int wdt, int ldw, int N, int K, int block, int8_t* Q,
                            int ldq, float* S, hipStream_t s);
int launch_gemm_i8(const int8_t* X, int ldx, const float* xs, const int8_t* W, int ldw,
                   const float* ws, int M, int N, int K, void* Y, int ldy, int ydt,
                   hipStream_t s);
void describe_i8(int M, int N, int K, char* buf, size_t len);

int launch_probe_read(const void* buf, size_t bytes, uint32_t* out,
                      hipStream_t s);
int launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t s);
int launch_probe_mfma(int iters, float* out, hipStream_t s);
size_t probe_handoff_bytes();
int launch_probe_handoff(void* work, int rounds, int rows, hipStream_t s);

}  // namespace w4
