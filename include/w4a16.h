/*
 * w4a16.h -- C ABI of libw4a16.so, an MI355X (gfx950) library for the W4A16
 * group-quantized matrix-vector product of batch-1 decode.
 *
 * Sources the operations follow (pages as published on the web):
 *  [P1] "Gemma 4 E2B on a 4 GB GPU with plain PyTorch, faster than llama.cpp"
 *       - the paragraph introducing the compressed-tensors W4A16 checkpoint:
 *         4-bit weights in groups of 32 with one 16-bit step (bf16) per group,
 *         16-bit activations;
 *       - the paragraph on the w4gemv.py kernel: decoding one token multiplies
 *         one vector by every weight matrix, so the speed limit is how fast
 *         the weights are read; the kernel reads the packed 4-bit words,
 *         unpacks them in registers and multiplies, never writing a 16-bit
 *         copy; each 4-bit value becomes the exact float (value - 8); each
 *         weight shape gets its own fixed tiling;
 *       - the paragraph on the decode step as one captured graph (launching
 *         hundreds of small kernels one at a time costs more than running
 *         them) and the paragraph on concatenated gate|up and q|k|v matrices;
 *       - the summary line of the kernel: GB/s counted from packed weight
 *         bytes, compared with a plain-sum read of memory.
 *  [P2] "fastgemma -- Gemma 4 E2B, CPU-only, AMX INT8 / AVX-512 VNNI"
 *       - section "What is in the file": int4 weights in groups of 256,
 *         rotated along K by an orthogonal Hadamard matrix (W' = W H^T) with a
 *         run-time fast Walsh-Hadamard transform of the activation; weights
 *         pre-packed once into the kernel's operand order;
 *       - section "Why AMX for GEMM but not for attention": a weight GEMM
 *         reuses each weight byte across all M activation rows.
 *
 * Conventions for every call:
 *  - Status: 0 (W4_OK) on success, a negative W4_ERR_* otherwise.  No call
 *    throws.  On a validation error nothing is launched and no output byte is
 *    written; w4_last_error() then holds a message for the calling thread.
 *  - Validation (shapes, group, dtype, null pointers, alignment) happens before
 *    any HIP call, so every error path can be exercised without a GPU.
 *  - Pointers named "device" are device (HBM) addresses, e.g. from hipMalloc or
 *    torch; "host" pointers are ordinary CPU memory.  The caller owns every
 *    buffer; the library never allocates on a compute call.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *    are stream-ordered and asynchronous: a launch failure returns W4_ERR_HIP,
 *    a fault shows at the caller's next synchronization.
 *  - Stateless calls are thread-safe.  A sweep handle is used by one thread.
 *
 * Weight format (canonical, what callers hold):
 *  - codes P[N][K/8] uint32: element (n, k) is the 4-bit code in word
 *    P[n][k/8], bits [4*(k%8), 4*(k%8)+4) (least significant nibble first);
 *  - scales S[N][K/group] bf16 (uint16 bit patterns), row-major;
 *  - weight value w(n,k) = (code - 8) * S[n][k/group] (offset binary, symmetric,
 *    no zero point).  A matrix is N x K like a linear layer's (out x in).
 * Device layout ("packed"), produced only by w4_pack / w4_pack_host and read
 * by every compute call: w4_packed_bytes(N, K, group) bytes holding the codes
 * (N*K/2 bytes, row-major, each word's nibbles reordered so that the codes of
 * elements 2j and 2j+1 sit at bits [4j, 4j+4) and [16+4j, 20+4j)), then, at the
 * next 256-byte boundary, the scales unchanged.  Callers treat it as opaque.
 * Activations X[M][K] are bf16, row stride ldx elements.  Outputs are fp32 or
 * bf16 (round to nearest even from the fp32 accumulator).
 *
 * Arithmetic of every product: each weight enters as the exact value
 * (code - 8), before it is multiplied ([P1], paragraph on the w4gemv.py
 * kernel), so a code of 8 contributes an exact zero; every product
 * (code - 8) * x is exact and only the fp32 sums round.  The batch-1 GEMV
 * scales each 32-element activation chunk by a power of two into fp16
 * (exact for chunks whose nonzero magnitudes lie within 2^29 of the largest,
 * and without inf / NaN; any other chunk sends its wave to an exact bf16
 * path); the matrix-core and small-M kernels keep the activations in bf16
 * and enter each code as the bf16 value 16 (code - 8).
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4_ABI_VERSION 1

enum w4_status {
    W4_OK = 0,
    W4_ERR_ARG = -1,          /* null pointer, bad enum, bad handle          */
    W4_ERR_SHAPE = -2,        /* N, K, M, group, block or size out of range  */
    W4_ERR_ALIGN = -3,        /* pointer or leading dimension misaligned     */
    W4_ERR_DTYPE = -4,        /* output dtype not W4_F32 / W4_BF16           */
    W4_ERR_UNSUPPORTED = -5,  /* valid request the library does not serve   */
    W4_ERR_HIP = -6,          /* a HIP runtime call failed                   */
    W4_ERR_NOMEM = -7,        /* allocation failed (sweep creation only)     */
    W4_ERR_ARCH = -8,         /* current device is not gfx950                */
    W4_ERR_TIMEOUT = -9,      /* a bounded in-kernel wait gave up            */
    W4_ERR_SELFTEST = -10     /* w4_selftest found a wrong output            */
};

enum w4_dtype { W4_F32 = 0, W4_BF16 = 1 };

/* Text for a status code (static storage). */
const char* w4_status_str(int status);

/* Detail of the last failed call on this thread ("" if none). */
const char* w4_last_error(void);

/* W4_OK if the current HIP device is gfx950, W4_ERR_ARCH otherwise,
 * W4_ERR_HIP if no device can be queried. */
int w4_device_check(void);

/* Library build information: "<abi version> <offload arch> <kernel set>". */
const char* w4_build_info(void);

/*
 * Bytes of the device layout for an N x K matrix (0 when the shape is
 * invalid: N < 1, K < 1, group not 32, 256 or 512, K % group != 0).
 */
size_t w4_packed_bytes(int N, int K, int group);

/*
 * Canonical (P, S) -> device layout, on the device.  P_canon: device,
 * N*K/8 uint32.  S_bf16: device, N*(K/group) uint16.  packed_out: device,
 * w4_packed_bytes(N, K, group) bytes, 16-byte aligned; must not overlap the
 * inputs.  [P2] "What is in the file": weights are packed once into the
 * kernel's load order so nothing is repacked at run time.
 */
int w4_pack(const uint32_t* P_canon, const uint16_t* S_bf16, int N, int K,
            int group, void* packed_out, void* stream);

/* Same transform on host memory (all three pointers host). */
int w4_pack_host(const uint32_t* P_canon, const uint16_t* S_bf16, int N,
                 int K, int group, void* packed_out);

/* Inverse of w4_pack_host: device layout (host copy) -> canonical P and S. */
int w4_unpack_host(const void* packed, int N, int K, int group,
                   uint32_t* P_canon, uint16_t* S_bf16);

/*
 * y = W x for one activation vector (M = 1): y[n] = sum_k w(n,k) x[k], fp32
 * accumulation, any summation order but bitwise run-to-run deterministic.
 * [P1] paragraph on the w4gemv.py kernel.
 *  packed: device layout of W (N x K, group 32, 256 or 512), 16-byte aligned.
 *  x: device, K bf16, 16-byte aligned.
 *  y: device, N elements of y_dtype (4-byte aligned for fp32, 2 for bf16);
 *     sharing no byte with x or packed (W4_ERR_ARG otherwise).
 * N >= 1; K >= 32 and K % group == 0.
 */
int w4a16_gemv(const void* packed, int N, int K, int group, const uint16_t* x,
               void* y, int y_dtype, void* stream);

/*
 * Y = X W^T for 2 <= M <= 16 activation rows, reading each weight byte once
 * for all M rows ([P2] "Why AMX for GEMM but not for attention": a weight GEMM
 * reuses each byte across all M rows).  When the activation rows fit a CU's
 * 160 KB of LDS and K % 128 == 0, one 16-row tile runs on the matrix cores
 * for groups 256 and 512, and for group 32 from 5 rows; other shapes run on
 * the vector ALU.
 *  X: device, M rows of K bf16, row stride ldx >= K elements (ldx % 8 == 0),
 *     16-byte aligned.
 *  Y: device, M rows of N y_dtype elements, row stride ldy >= N elements;
 *     its span shares no byte with X's span or packed (W4_ERR_ARG otherwise).
 */
int w4a16_gemm_smallM(const void* packed, int N, int K, int group, int M,
                      const uint16_t* X, int ldx, void* Y, int ldy,
                      int y_dtype, void* stream);

/*
 * Blockwise fast Walsh-Hadamard transform of activations along K ([P2]
 * "What is in the file"): every contiguous block of `block` elements of each
 * row is multiplied by the Sylvester-ordered Hadamard matrix of that size
 * scaled by block^-1/2 (orthonormal).  fp32 arithmetic, bf16 result (round to
 * nearest even).  block is a power of two, 2 <= block <= 1024, K % block == 0.
 *  X: device, M x K bf16, stride ldx (>= K, % 8 == 0).  Xout: device, stride
 *  ldo.  Xout may equal X (in place) when ldo == ldx.
 */
int w4_fwht(const uint16_t* X, int ldx, uint16_t* Xout, int ldo, int M, int K,
            int block, void* stream);

/* Workspace bytes w4a16_gemm needs (0 when had_block == 0). */
size_t w4a16_gemm_workspace_bytes(int M, int K, int had_block);

/*
 * Y = X' W'^T, the prefill-shaped product on the matrix cores (bf16 MFMA,
 * fp32 accumulation): X' = X when had_block == 0, else X' is the blockwise
 * FWHT of X (block had_block, computed into `workspace`, M*K bf16) and W' is
 * stored pre-rotated.  [P2] "fastgemma -- Gemma 4 E2B, CPU-only, AMX INT8 /
 * AVX-512 VNNI": section "What is in the file" (int4 groups of 256, Hadamard
 * rotation W' = W H^T with a run-time FWHT of the activation) and section
 * "Why AMX for GEMM but not for attention" (a weight GEMM reuses every weight
 * byte across all M rows, so at prefill row counts the multiply units, not
 * memory, bound it).  Codes enter the matrix cores as the exact bf16 values
 * 16 (code - 8); each K-group's partial product is multiplied by its fp32
 * scale / 16.
 *  group must be 256 or 512 (the rotated prefill format of [P2]) or 32.
 *  M >= 1, K % 256 == 0.  Decode-shaped row counts take the decode kernels
 *  after the same transform: M = 1 the GEMV.  2..32 rows (8..32 at group
 *  32) of a matrix of at least 128 tiles of 48 rows with K a multiple of
 *  512 up to 2048 run on the split-K matrix-core kernel (K in four slices
 *  per workgroup, the sum of the slices in a fixed order).  Otherwise 2..8
 *  rows take the small-M product, and 9..16 too where it runs on the
 *  matrix cores (see w4a16_gemm_smallM); larger row counts run on the tiled
 *  matrix-core kernels.
 *  X: device, stride ldx (% 8 == 0).  Y: device, stride ldy; its span
 *  shares no byte with X's span or packed (W4_ERR_ARG otherwise).
 *  workspace: device, >= w4a16_gemm_workspace_bytes(M, K, had_block) bytes,
 *  16-byte aligned (may be NULL when that size is 0).
 */
int w4a16_gemm(const void* packed, int N, int K, int group, int M,
               const uint16_t* X, int ldx, int had_block, void* workspace,
               size_t ws_bytes, void* Y, int ldy, int y_dtype, void* stream);

/*
 * w4a16_gemm for callers that cannot allocate memory (code under graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * product and kernels, but the transform's output (when had_block != 0) is
 * written to a fixed 8 MiB device array of this library instead of a caller
 * workspace, so the call allocates nothing.  Each GPU holds its own copy of
 * that array until the process ends; its device address is looked up once
 * per device on the first call made with that device current.
 *  Size limit: M * K * 2 bytes (rounded up to 256) must not exceed
 *  w4a16_gemm_noalloc_max_bytes() when had_block != 0; larger calls return
 *  W4_ERR_SHAPE before any HIP call.  Every other argument as w4a16_gemm.
 *  Calls that overlap on one GPU (on different streams, or from several
 *  threads) share the array and race; serialize them.  The array keeps the
 *  last call's transform output; nothing in it needs to start at zero.
 */
int w4a16_gemm_noalloc(const void* packed, int N, int K, int group, int M,
                       const uint16_t* X, int ldx, int had_block, void* Y, int ldy,
                       int y_dtype, void* stream);
/* Bytes of the static transform array (8 MiB). */
size_t w4a16_gemm_noalloc_max_bytes(void);

/*
 * A decode step's worth of GEMVs replayed as one unit ([P1] paragraph on the
 * decode step captured once as a graph and replayed per token).
 * Each op is one w4a16_gemv (M = 1).  The handle owns its graph, its
 * executable graph and a small device buffer (op table, counters, flags); it
 * BORROWS every pointer in `ops`, which must stay valid while the handle
 * lives.  Ops run in array order.  No op's y may share a byte with its own
 * x or with any op's weights (W4_ERR_ARG); an op's x may be an earlier op's
 * y (the decode-ordered mode orders them).
 * Modes:
 *  W4_SWEEP_GRAPH      one GEMV kernel per op captured into a hipGraph;
 *                      op i+1 starts after op i has finished (stream order).
 *  W4_SWEEP_PERSISTENT one persistent kernel (one workgroup per CU) walks all
 *                      ops in order; each workgroup's share of the next op's
 *                      weights is loaded into LDS ahead of time (weights never
 *                      depend on activations), but no output of op i+1 is
 *                      computed, and no activation of op i+1 is read, before
 *                      every output of op i is written: the ordering of a
 *                      decode step, so op i+1 may read op i's output.
 *                      Replays of one handle must not overlap (the handle's
 *                      counters serve one replay at a time), and the kernel
 *                      needs every workgroup resident at once (nothing else
 *                      occupying the CUs).  Bounded waits: a wait that exceeds
 *                      its limit ends the kernel and is reported by
 *                      w4_decode_sweep_check as W4_ERR_TIMEOUT (the check then
 *                      resets the handle's counters).
 *  W4_SWEEP_STREAM     the persistent kernel without the op-to-op ordering
 *                      (ops treated as independent); an upper bound.
 * The persistent modes are one kernel launch per replay.
 */
typedef struct w4_gemv_op {
    const void* packed;      /* device layout of this op's weights   */
    int N, K, group;         /* shape; group 32, 256 or 512          */
    const uint16_t* x;       /* device, K bf16, 16-byte aligned      */
    void* y;                 /* device, N elements of y_dtype        */
    int y_dtype;             /* W4_F32 or W4_BF16                    */
} w4_gemv_op;

enum w4_sweep_mode {
    W4_SWEEP_GRAPH = 0,
    W4_SWEEP_PERSISTENT = 1,
    W4_SWEEP_STREAM = 2
};

typedef struct w4_sweep w4_sweep;

/* Validates every op and builds the replay: the graph of per-op kernels
 * (GRAPH) or the persistent kernel's op table (other modes).  `stream` is
 * unused (setup is synchronous). */
int w4_decode_sweep_create(const w4_gemv_op* ops, int n_ops, int mode,
                           void* stream, w4_sweep** out);
/* One replay on `stream`: one hipGraphLaunch (GRAPH) or one kernel launch
 * (other modes).  May be recorded into a caller's graph capture. */
int w4_decode_sweep_launch(w4_sweep* h, void* stream);
/* Synchronizes `stream` and reports a timed-out wait of a persistent replay
 * since the last check (W4_ERR_TIMEOUT), else W4_OK. */
int w4_decode_sweep_check(w4_sweep* h, void* stream);
/* Number of ops, total algorithmic weight bytes, kernels per replay. */
int w4_decode_sweep_info(const w4_sweep* h, int* n_ops, size_t* weight_bytes,
                         int* kernels_per_replay);
int w4_decode_sweep_destroy(w4_sweep* h);

/*
 * Rotate-and-quantize: dense weights -> the device layout, on the GPU.
 * [P2] section "What is in the file": every linear weight is rotated along K
 * by an orthogonal Hadamard matrix, W' = W H^T, and stored as int4 with one
 * scale per group (group 256 there); with the run-time transform of the
 * activation (w4_fwht, or had_block of w4a16_gemm) the product is unchanged,
 * and groups with outliers quantize with less error.  The page gives no
 * scale rule; the rule here is symmetric per group:
 *   s = bf16(max|w'| / 7)  (round to nearest even),
 *   q = clamp(round_half_even(w' / s), -8, 7),  code = q + 8,
 * with s = 0 and code 8 for an all-zero group; the rotation (butterfly
 * stages of span 1, 2, 4, ..., then one fp32 scaling by block^-1/2) and every
 * rounding decision are fp32, so the output is a deterministic function of W.
 *  W:        device, N rows of ldw elements (ldw >= K), fp32 or bf16
 *            (w_dtype W4_F32 / W4_BF16), 16-byte aligned, each row 16-byte
 *            aligned (ldw % 4 == 0 for fp32, % 8 for bf16); finite values.
 *  had_block: 0 (no rotation) or 64, 128, 256, 512 (Sylvester order,
 *            orthonormal, contiguous blocks along K; K % had_block == 0).
 *  packed:   device, w4_packed_bytes(N, K, group) bytes, 16-byte aligned;
 *            written completely (codes and scales).
 */
int w4_quantize(const void* W, int w_dtype, int ldw, int N, int K, int group,
                int had_block, void* packed, void* stream);

/*
 * The int8 twin ([P2] section "What is in the file": the FFN weights are
 * also kept as int8, twice the int4 bytes; prefill runs on int8, selected
 * automatically at 16 rows or more -- FGM_WEIGHTS=auto:16 -- decode on
 * int4).  Both operands of the int8 product are int8: weights per output
 * channel, activations per row at run time.  Rule (the page gives none):
 * after an optional rotation (had_block, as w4_quantize), each row gets an
 * fp32 scale s = max|v| / 127 and codes q = clamp(round_half_even(v / s),
 * -127, 127), all in fp32.
 *
 * w4_quantize_rows_i8: N rows of X (fp32 or bf16, ldx >= K, 16-byte aligned
 *   rows) -> Q int8 [N][ldq] (ldq >= K, ldq % 8 == 0, Q 16-byte aligned;
 *   ldq % 16 == 0 for rows w4_gemm_i8 reads) and S fp32 [N].  K % 8 == 0.
 *   Used offline for the weight twin and at run time for activations.
 * w4_gemm_i8: Y[m][n] = (sum_k Xq[m][k] Wq[n][k]) * xs[m] * ws[n] on the int8
 *   matrix cores (exact int32 sums; the int32 -> fp32 conversion and the two
 *   scale multiplications round in fp32).  K % 128 == 0; Xq, Wq rows 16-byte
 *   aligned (ldx, ldw >= K and % 16); Y fp32 or bf16 (nearest even), ldy >= N.
 * w4a16_gemm_twin: the auto:M switch.  M < switch_rows (the page: 16): the
 *   int4 product w4a16_gemm on packed4; otherwise the activations are
 *   rotated and quantized into the workspace and multiplied by the int8
 *   twin (W8 [N][ldw8], ws8 [N], quantized from the same weights with the
 *   same had_block).  workspace >= w4a16_gemm_twin_workspace_bytes(M, K,
 *   had_block, switch_rows), 16-byte aligned.
 */
int w4_quantize_rows_i8(const void* X, int x_dtype, int ldx, int N, int K,
                        int had_block, int8_t* Q, int ldq, float* S,
                        void* stream);
int w4_gemm_i8(const int8_t* Xq, int ldx, const float* xs, const int8_t* Wq,
               int ldw, const float* ws, int M, int N, int K, void* Y,
               int ldy, int ydt, void* stream);
size_t w4a16_gemm_twin_workspace_bytes(int M, int K, int had_block,
                                       int switch_rows);
int w4a16_gemm_twin(const void* packed4, const int8_t* W8, int ldw8,
                    const float* ws8, int N, int K, int group, int M,
                    const uint16_t* X, int ldx, int had_block, int switch_rows,
                    void* workspace, size_t ws_bytes, void* Y, int ldy,
                    int ydt, void* stream);

/*
 * Split-K decode attention: one key/value head shared by 8 query heads.
 * [P1] paragraph on w4attn.py: each cached key and value is read once for
 * all eight query heads, the cache is split into slices and the slices are
 * combined with an online softmax; paragraph on the cache: full layers hold
 * one slot per position (head width 512), sliding layers a 512-slot ring
 * recording each slot's position, masks built from positions.
 *   valid(t) = t < T and (pos == NULL or (pos[t] >= 0 and pos[t] <= cur and
 *              (window == 0 or pos[t] > cur - window)))
 *   s_t = scale * q_h . K[t],  out[h] = sum_t softmax_t(s) V[t]  over valid t.
 *  q:   device, [8][D] bf16, 16-byte aligned.
 *  K:   device, T rows of ldk bf16 (ldk >= D, ldk % 8 == 0), 16-byte aligned.
 *  Vt:  device, V in the blocked layout: ceil(T/32) blocks of 32 slots, block
 *       b holding D rows of 32 bf16; slot t, dim d at Vt[((t/32)*D + d)*32 +
 *       t%32].  w4_attn_pack_v writes it from row-major V; w4_attn_store_kv
 *       writes one slot.  Slots that are not valid may hold any bits.
 *  pos: NULL (slots 0..T-1 all valid: a full-length cache) or device int32
 *       [T] slot positions (-1 = empty), e.g. a ring of 512 slots.
 *  D:   256 or 512.  T: 1 .. 2^24 slots scanned.  window >= 0.  scale finite.
 *  workspace: device, >= w4_attn_workspace_bytes(T, D) bytes, 16-byte aligned
 *       (per-slice partials; overwritten).
 *  out: device, [8][D] fp32 or bf16 (nearest even), 16-byte aligned.  A head
 *       with no valid slot gets NaN.
 * Products on the matrix cores (bf16 operands, fp32 accumulation); the
 * softmax weights enter the value product as bf16 (nearest even) and the
 * normaliser sums those same weights.  Two launches (split, merge).
 */
size_t w4_attn_workspace_bytes(int T, int D);
int w4_attn_decode(const uint16_t* q, const uint16_t* K, int ldk,
                   const uint16_t* Vt, const int32_t* pos, int T, int D,
                   int cur, int window, float scale, void* workspace,
                   size_t ws_bytes, void* out, int out_dtype, void* stream);
/* Row-major V (T rows of ldv bf16, ldv >= D) -> the blocked layout above
 * (ceil(T/32)*32*D bf16; slots past T written as 0).  Vt 16-byte aligned. */
int w4_attn_pack_v(const uint16_t* V, int ldv, int T, int D, uint16_t* Vt,
                   void* stream);
/* One decode step's cache write: K[slot] = k (D bf16), V slot `slot` = v,
 * in the blocked layout. */
int w4_attn_store_kv(const uint16_t* k, const uint16_t* v, int slot,
                     uint16_t* K, int ldk, uint16_t* Vt, int D, void* stream);

/*
 * Row lookup in a 4-bit table, dequantized:
 *   Y[b][k] = (code(ids[b], k) - 8) * scale(ids[b], k / group),  b < B, k < K.
 * [P1] step 2 "Keep the Vocabulary Tables in 4-Bit": the token-embedding
 * table (the same copy serves as the output layer, whose GEMV is w4a16_gemv)
 * and the per-layer input table (a row of 35 x 256 values per token) are
 * 4-bit codes with a 16-bit step per group, looked up on the GPU.
 *  packed: device layout (w4_pack) of the N x K table, 16-byte aligned.
 *  ids:    device, B int32 row indices, 4-byte aligned; duplicates allowed.
 *          An id outside [0, N) reads nothing and yields a row of quiet NaNs.
 *  Y:      device, B rows of ldy elements (ldy >= K), 16-byte aligned, each
 *          row 16-byte aligned (ldy % 4 == 0 for fp32, % 8 for bf16).
 *  ydt:    W4_F32 (exact: the values have at most 12 significant bits) or
 *          W4_BF16 (round to nearest even).
 * B = 0 is a no-op; B <= 2^24.
 */
int w4_gather(const void* packed, int N, int K, int group, const int32_t* ids,
              int B, void* Y, int ldy, int ydt, void* stream);

/*
 * The kernel and tile the dispatcher picks for (M, N, K, group), as text
 * (e.g. "gemv L=16 U=3 W=4 grid=160 stages=2 (built-in table)"), written
 * NUL-terminated into buf (truncated to len - 1 characters).  [P1] paragraph
 * on the w4gemv.py kernel: each weight shape gets its own fixed tiling, found
 * by searching tile sizes, warps and pipeline stages on the card.
 */
int w4_describe_dispatch(int M, int N, int K, int group, char* buf,
                         size_t len);

/*
 * Run-time dispatch configuration.  Read from the environment on the first
 * dispatching call and again by w4_config_reload():
 *  W4_TILE_TABLE=path   a batch-1 GEMV tile table (format below) whose
 *                       entries replace the built-in table's for their
 *                       shapes.  A file that cannot be read or has any bad
 *                       line is rejected as a whole: every dispatching call
 *                       then returns its status (W4_ERR_ARG or W4_ERR_SHAPE)
 *                       with the file, line and reason in w4_last_error().
 *  W4_FORCE_PATH=a,b    force kernel families wherever they apply:
 *                       gemv_generic, gemv_tiled (heuristic tile, no table),
 *                       gemv_contig (heuristic tile, contiguous row ranges
 *                       where the tile allows), smallm_valu (vector-ALU
 *                       small-M kernel), prefill_regs (register-staged
 *                       matrix-core kernel), i8_regs (register-staged int8
 *                       kernel), ordered_inline (decode-ordered sweep:
 *                       decode each share while multiplying instead of
 *                       ahead), no_splitk (w4a16_gemm: not the split-K
 *                       kernel; smallm_valu and prefill_regs also keep it
 *                       off the row counts they name).  An unknown name is
 *                       W4_ERR_ARG.
 *  W4_LOG=1             print each distinct dispatch decision once to stderr.
 *  W4_SWEEP_POLL_LIMIT=n
 *                       completion polls per op before a decode-ordered
 *                       sweep handle created afterwards gives up (default
 *                       2^20); 0 makes every replay give up at its second
 *                       op, for tests of the W4_ERR_TIMEOUT path.
 *  W4_SWEEP_BLOCKS_PER_CU=n (1..16)
 *                       workgroups per CU of an unordered (STREAM) sweep
 *                       handle created afterwards (default 5, capped at what
 *                       fits a CU at once), for tuning runs; read when the
 *                       handle is created.
 *  W4_PREFILL_CFG, W4_MFMA_CFG, W4_I8_RING (1..4), W4_I8_TILE ("MF,NF"):
 *                       tiling indices of the prefill, register-staged
 *                       matrix-core and int8 kernels, for tuning runs.
 * Batch-1 GEMV tile order: W4_FORCE_PATH, the loaded table, the built-in
 * table (searched on MI355X for the model's shapes), the heuristic.
 *
 * Tile table format: text, one entry per line, '#' starts a comment:
 *   gemv N K group L U waves grid stages contig
 *  L       lanes per row: 8, 16, 32 or 64
 *  U       32-element chunks per lane, ceil(K / 32 / L) (the register-tiled
 *          loop; needs an even K / group), or 0 for the generic loop
 *  waves   waves per workgroup, 1..4
 *  grid    workgroups, 1..65535, or 0 to derive it from the shape
 *  stages  row groups in flight + 1: 2, or 3 with 1 <= U <= 4
 *  contig  1: every wave streams one contiguous range of rows (needs
 *          L >= 16, L U = K / 32, U <= 3 and 4 waves), 0: rows strided over
 *          the grid
 * A shape may appear once; at most 4096 entries, 1 MiB.
 */
int w4_config_reload(void);

/* Replaces the loaded tile table with the file at `path` (validated as
 * above; on error the previous table stays), or removes it (path NULL).
 * Takes precedence over W4_TILE_TABLE until the next w4_config_reload(). */
int w4_tile_table_load(const char* path);

/*
 * Start-up check of the compute paths on the current device ([P2] probes its
 * machine at start-up before trusting a kernel path).  Runs the batch-1 GEMV
 * (group 32 and 256), the small-M kernel (M = 8) and the matrix-core GEMM
 * (M = 64) through the public entry points on built-in 100 x 512 matrices
 * with one-hot activations, whose outputs are exactly (code - 8) * scale, and
 * compares every output bitwise.  Allocates and frees about 1 MB of device
 * memory and synchronizes `stream` (not for use inside a graph capture).
 * W4_OK; W4_ERR_SELFTEST with the first wrong output in w4_last_error();
 * W4_ERR_ARCH / W4_ERR_HIP / W4_ERR_NOMEM as for other calls.
 */
int w4_selftest(void* stream);

/*
 * Plain-sum read of `bytes` of device memory (the measurement the summary line
 * of [P1]'s kernel compares against): *out = sum of the buffer's 32-bit words
 * as unsigned integers modulo 2^32 (integer sum, so the result does not depend
 * on the order of reads).  buf: device, 16-byte aligned, bytes % 16 == 0,
 * bytes > 0.  out: device, one uint32, 4-byte aligned.
 */
int w4_probe_read(const void* buf, size_t bytes, uint32_t* out, void* stream);

/* Plain copy of `bytes` (16-byte aligned pointers, bytes % 16 == 0): the
 * reference kernel for calibrating hardware byte counters. */
int w4_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

/*
 * Matrix-core throughput probe (the measured ceiling the prefill products are
 * compared with): 512 workgroups of four waves, two waves per SIMD, each wave
 * running `iters` rounds of 16 independent v_mfma_f32_16x16x32_bf16 chains
 * from registers; 2 * 16 * 16 * 32 = 16384 FLOP per MFMA, so one call does
 * 2048 waves * iters * 16 * 16384 FLOP.  Nothing is written (out is touched
 * only if the positive sum turned negative).  iters in 1..2^20.  out: device,
 * 4-byte aligned, not NULL.
 */
int w4_probe_mfma(int iters, float* out, void* stream);

/*
 * Grid-wide handoff probe: the fixed cost each op of the decode-ordered sweep
 * pays because it reads the whole output of the op before it ([P1], paragraph
 * on the decode step captured once as a graph: every GEMV of a step reads
 * what the previous one wrote), measured with no weights.  One workgroup of
 * one wave per CU (256) runs `rounds` rounds; in each, every workgroup
 * stores `rows` bf16 values (its share of a vector of 256 * rows elements)
 * at agent scope, waits for them to complete, adds one to its XCD's
 * completion counter, polls the eight counters until every workgroup has
 * signalled, then loads the whole vector into LDS (agent scope, 16-byte
 * global-to-LDS loads) and waits for it, as the sweep kernel's control wave
 * does before each op.  rows = 0 times the bare signal-and-poll round.  The
 * caller times the call (two round counts, the difference over the extra
 * rounds, removes the launch).  Round r writes the value r + j (as a 16-bit
 * integer) at element w * rows + j of buffer r mod 2.
 *  work: device, >= w4_probe_handoff_bytes() bytes, 256-byte aligned.
 *  Layout: 512 control words (word 0 is nonzero afterwards if a poll gave
 *  up), then the two vectors of 256 * 64 elements each.  The call clears the
 *  control words with hipMemsetAsync first, so it is not for graph capture.
 *  rounds in 1..2^20, rows in 0..64.
 */
size_t w4_probe_handoff_bytes(void);
int w4_probe_handoff(void* work, int rounds, int rows, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
