/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar CPU reference for the W4A16 group-quantized
 * matrix-vector / matrix-matrix product and the blockwise Walsh-Hadamard
 * transform of activations.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the GPU library: everything below is written
 * from the definitions on the pages, in fp64, in the order they state.
 *
 * Sources (pages as published on the web):
 *  [P1] "Gemma 4 E2B on a 4 GB GPU with plain PyTorch, faster than llama.cpp":
 *       - paragraph introducing the compressed-tensors W4A16 checkpoint:
 *         4-bit weights in groups of 32, one 16-bit (bf16) step per group,
 *         16-bit activations;
 *       - paragraph on the w4gemv.py kernel: decoding one token multiplies one
 *         vector by every weight matrix; the kernel reads the packed 4-bit
 *         words and multiplies, and each 4-bit value becomes a float as
 *         (value - 8), exactly.
 *  [P2] "fastgemma -- Gemma 4 E2B, CPU-only, AMX INT8 / AVX-512 VNNI",
 *       section "What is in the file": weights rotated along K by an orthogonal
 *       Hadamard matrix H, W' = W H^T, and a fast Walsh-Hadamard transform of
 *       the activation at run time gives the same product; FFN weights are
 *       int4 with groups of 256.
 *
 * Readings where the pages are silent (each is also listed in the design
 * notes of the repository):
 *  - nibble order: element k of a row sits in word k/8, bits [4*(k%8), +4),
 *    least significant nibble first;
 *  - sign convention: offset binary, value = (code - 8) * scale (not two's
 *    complement int4);
 *  - scales: S[n][k / group], row-major, bf16, no zero point;
 *  - Hadamard: Sylvester (natural) order, orthonormal factor block^-1/2,
 *    contiguous blocks along K; Sylvester H is symmetric, so H^T = H;
 *  - bf16 outputs: round to nearest, ties to even.
 *
 * Rotate-and-quantize: [P2] section "What is in the file": every linear
 * weight is rotated along K by the orthogonal Hadamard matrix, W' = W H^T,
 * and stored as int4 with one scale per group; the pages do not give the
 * scale rule.  Reading taken: symmetric, s = bf16(max|w'| / 7) per group,
 * q = clamp(round_half_even(w' / s), -8, 7), code = q + 8; all-zero groups
 * get s = 0 and code 8.  The rotation and the rounding decisions are made in
 * fp32, the kernel's precision, so that both sides decide every code alike.
 *
 * int8 twin: [P2] section "What is in the file": the FFN weights are also
 * stored as an int8 twin (per output channel), and prefill runs on int8
 * ("selected automatically at >= 16 rows", the auto:M switch), decode on
 * int4.  Both operands of the pages' int8 product are int8, so the
 * activations are quantized at run time too.  Reading taken (the rule is not
 * given): every row (of W', and of the rotated activations x') is quantized
 * symmetrically with its own fp32 scale s = max|v| / 127,
 * q = clamp(round_half_even(v / s), -127, 127); the product is the exact
 * integer sum times both scales.
 *
 * Decode attention: [P1] paragraph on w4attn.py: one key/value head is shared
 * by eight query heads; every cached key and value is read once for all
 * eight heads and the softmax runs over the cache; paragraph on the cache:
 * full layers hold one slot per position, sliding layers a 512-slot ring that
 * records each slot's position, and masks come from positions.  The oracle is
 * the definition: scores s_t = scale * q.k_t over the valid slots, softmax,
 * output sum_t p_t v_t, in fp64.
 *
 * Table gather: [P1], step 2 "Keep the Vocabulary Tables in 4-Bit": the
 * token-embedding table (one copy, shared with the output layer) and the
 * per-layer input table (a row of 35 x 256 values per token) are stored as
 * 4-bit codes with one 16-bit step per group, and the row lookup runs on the
 * GPU; a looked-up row is the dequantized row w(id, k), k = 0..K-1.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 is the top 16 bits of an IEEE binary32; widening is exact. */
double oracle_bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

void oracle_bf16_array_to_f64(const uint16_t* in, double* out, size_t n)
{
    for (size_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_f64(in[i]);
}

/* The 4-bit code of element (n, k) of an N x K matrix whose canonical packed
 * form is P[N][K/8] (uint32), integer arithmetic only. */
int oracle_code(const uint32_t* P, int K, int n, int k)
{
    const uint32_t word = P[(size_t)n * (size_t)(K / 8) + (size_t)(k / 8)];
    const int shift = 4 * (k % 8);
    return (int)((word >> shift) & 0xFu);
}

/* All codes, row-major N x K, as small integers 0..15. */
void oracle_codes(const uint32_t* P, int N, int K, int8_t* out)
{
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k)
            out[(size_t)n * K + k] = (int8_t)oracle_code(P, K, n, k);
}

/* Dequantized weight value (code - 8) * scale, exact in fp64
 * (a 4-bit integer times an 8-significant-bit scale). */
double oracle_weight(const uint32_t* P, const uint16_t* S, int K, int group, int n, int k)
{
    const int v = oracle_code(P, K, n, k) - 8;
    const double s = oracle_bf16_to_f64(S[(size_t)n * (size_t)(K / group) + (size_t)(k / group)]);
    return (double)v * s;
}

void oracle_dequant(const uint32_t* P, const uint16_t* S, int N, int K, int group, double* W)
{
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k)
            W[(size_t)n * K + k] = oracle_weight(P, S, K, group, n, k);
}

/*
 * Y[m][n] = sum_{k=0..K-1} w(n,k) * X[m][k], summed in order of increasing k
 * in fp64; A[m][n] = sum_k |w(n,k) * X[m][k]| (the scale of the acceptance
 * bound).  X is fp64 (the caller widens bf16 activations exactly, or passes a
 * Hadamard-transformed activation).  Rows of X are ldx apart.
 * nthreads > 1 splits the independent output rows n over OpenMP threads; the
 * arithmetic of each output is unchanged.
 */
void oracle_gemm(const uint32_t* P, const uint16_t* S, int N, int K, int group,
                 const double* X, int M, int ldx, double* Y, double* A, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    for (int m = 0; m < M; ++m) {
        const double* x = X + (size_t)m * (size_t)ldx;
#pragma omp parallel for num_threads(nthreads) schedule(static)
        for (int n = 0; n < N; ++n) {
            double y = 0.0, a = 0.0;
            for (int k = 0; k < K; ++k) {
                const double t = oracle_weight(P, S, K, group, n, k) * x[k];
                y += t;
                a += fabs(t);
            }
            Y[(size_t)m * N + n] = y;
            if (A) A[(size_t)m * N + n] = a;
        }
    }
}

/*
 * Blockwise fast Walsh-Hadamard transform along K, one row of X at a time:
 * every contiguous block of `block` (a power of two) elements is replaced by
 * H_block times that block, H_block the Sylvester-ordered Hadamard matrix
 * scaled by block^-1/2 (orthonormal).  Butterfly stages of span 1, 2, 4, ...
 * (a, b) -> (a + b, a - b), then one scaling.  K must be a multiple of block.
 */
void oracle_fwht(const double* X, double* Xout, int M, int K, int block)
{
    const double norm = 1.0 / sqrt((double)block);
    for (int m = 0; m < M; ++m) {
        const double* x = X + (size_t)m * K;
        double* y = Xout + (size_t)m * K;
        for (int k = 0; k < K; ++k) y[k] = x[k];
        for (int b0 = 0; b0 < K; b0 += block) {
            double* v = y + b0;
            for (int h = 1; h < block; h *= 2) {
                for (int i = 0; i < block; i += 2 * h) {
                    for (int j = i; j < i + h; ++j) {
                        const double a = v[j];
                        const double b = v[j + h];
                        v[j] = a + b;
                        v[j + h] = a - b;
                    }
                }
            }
            for (int j = 0; j < block; ++j) v[j] *= norm;
        }
    }
}

/*
 * fp64 -> bf16 bit pattern, round to nearest, ties to even, written from the
 * definition: with |v| = m * 2^e (0.5 <= m < 1), bf16 keeps 8 significant
 * bits, so the two neighbours of |v| are floor(m * 2^8) and that + 1, in units
 * of 2^(e-8); the nearer is taken, and on a tie the even one.  v must be zero
 * or have a magnitude in bf16's normal range (every value the gather makes
 * from a normal bf16 scale does).
 */
uint16_t oracle_f64_to_bf16(double v)
{
    if (v == 0.0) return signbit(v) ? 0x8000u : 0u;
    int e;
    const double m = frexp(fabs(v), &e);
    const double t = ldexp(m, 8);          /* 128 <= t < 256 */
    const double lo = floor(t);
    const double dlo = t - lo, dhi = lo + 1.0 - t;
    double r;
    if (dlo < dhi)
        r = lo;
    else if (dhi < dlo)
        r = lo + 1.0;
    else
        r = fmod(lo, 2.0) == 0.0 ? lo : lo + 1.0;
    const float f = (float)ldexp(r, e - 8);  /* <= 8 significant bits: exact */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t h = (uint16_t)(u >> 16);
    if (v < 0.0) h |= 0x8000u;
    return h;
}

/*
 * Rows ids[0..B-1] of an N x K table, dequantized: Y[b][k] = w(ids[b], k).
 * out_bf16 = 0: Y is float[B][K], each value exact ((code - 8) * scale has at
 * most 12 significant bits); out_bf16 = 1: Y is uint16[B][K], bf16 rounded to
 * nearest even.  An id outside [0, N) gives a row of quiet NaNs.
 */
void oracle_gather(const uint32_t* P, const uint16_t* S, int N, int K, int group,
                   const int32_t* ids, int B, int out_bf16, void* Y)
{
    for (int b = 0; b < B; ++b) {
        const int id = ids[b];
        for (int k = 0; k < K; ++k) {
            const size_t at = (size_t)b * K + k;
            if (id < 0 || id >= N) {
                if (out_bf16)
                    ((uint16_t*)Y)[at] = 0x7FC0u;
                else
                    ((float*)Y)[at] = (float)NAN;
                continue;
            }
            const double w = oracle_weight(P, S, K, group, id, k);
            if (out_bf16)
                ((uint16_t*)Y)[at] = oracle_f64_to_bf16(w);
            else
                ((float*)Y)[at] = (float)w;
        }
    }
}

/*
 * Rotate (optionally) and quantize an N x K fp32 matrix W (rows ldw apart)
 * into canonical codes P[N][K/8] and bf16 scales S[N][K/group].
 * block = 0: no rotation; otherwise each contiguous block of `block` elements
 * of a row becomes H_block times it, computed in fp32 by butterfly stages of
 * span 1, 2, 4, ... ((a, b) -> (a + b, a - b)) and one multiplication by
 * (float)(block^-1/2).  Then per group of `group` elements:
 *   a = max |w'| (fp32), s = a / 7 (fp32 division), sb = bf16 of s (nearest
 *   even), sf = sb widened; q = sf == 0 ? 0 : rint(w' / sf) (fp32 division,
 *   round half to even), clamped to [-8, 7]; code = q + 8.
 * Scales must come out zero or bf16-normal (true for any W whose group maxima
 * exceed 7 * 2^-126).
 */
void oracle_quantize(const float* W, int N, int K, int ldw, int group, int block,
                     uint32_t* P, uint16_t* S)
{
    float* v = (float*)malloc(sizeof(float) * (size_t)K);
    const float norm = block ? (float)(1.0 / sqrt((double)block)) : 1.0f;
    for (int n = 0; n < N; ++n) {
        for (int k = 0; k < K; ++k) v[k] = W[(size_t)n * ldw + k];
        if (block) {
            for (int b0 = 0; b0 < K; b0 += block) {
                float* x = v + b0;
                for (int h = 1; h < block; h *= 2)
                    for (int i = 0; i < block; i += 2 * h)
                        for (int j = i; j < i + h; ++j) {
                            const float a = x[j], b = x[j + h];
                            x[j] = a + b;
                            x[j + h] = a - b;
                        }
                for (int j = 0; j < block; ++j) x[j] = x[j] * norm;
            }
        }
        for (int k = 0; k < K / 8; ++k) P[(size_t)n * (K / 8) + k] = 0u;
        for (int g0 = 0; g0 < K; g0 += group) {
            float a = 0.0f;
            for (int k = g0; k < g0 + group; ++k)
                if (fabsf(v[k]) > a) a = fabsf(v[k]);
            const float sc = a / 7.0f;
            const uint16_t sb = oracle_f64_to_bf16((double)sc);
            const float sf = (float)oracle_bf16_to_f64(sb);
            S[(size_t)n * (K / group) + g0 / group] = sb;
            for (int k = g0; k < g0 + group; ++k) {
                float q = 0.0f;
                if (sf != 0.0f) {
                    q = rintf(v[k] / sf);
                    if (q < -8.0f) q = -8.0f;
                    if (q > 7.0f) q = 7.0f;
                }
                const uint32_t code = (uint32_t)((int)q + 8);
                P[(size_t)n * (K / 8) + k / 8] |= code << (4 * (k % 8));
            }
        }
    }
    free(v);
}

/*
 * Decode attention, one KV head, H query heads, head width D, T cache slots:
 *   valid(t) = pos == NULL ? 1
 *              : pos[t] >= 0 && pos[t] <= cur && (window <= 0 || pos[t] > cur - window)
 *   s_t = scale * sum_d q[h][d] K[t][d]   (valid t), m = max_t s_t,
 *   p_t = exp(s_t - m), out[h][d] = sum_t p_t V[t][d] / sum_t p_t,
 *   absout[h][d] = sum_t p_t |V[t][d]| / sum_t p_t  (scale of the acceptance bound).
 * q, K, V are bf16 bit patterns (row-major, rows of D), widened exactly; all
 * sums in fp64, in order of increasing t.  No valid slot: NaN outputs.
 */
void oracle_attn_decode(const uint16_t* q, const uint16_t* K, const uint16_t* V,
                        const int32_t* pos, int H, int T, int D, int cur, int window,
                        double scale, double* out, double* absout)
{
    double* sc = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    for (int h = 0; h < H; ++h) {
        double m = -INFINITY;
        int any = 0;
        for (int t = 0; t < T; ++t) {
            int ok = 1;
            if (pos) ok = pos[t] >= 0 && pos[t] <= cur && (window <= 0 || pos[t] > cur - window);
            if (!ok) {
                sc[t] = -INFINITY;
                continue;
            }
            double d = 0.0;
            for (int k = 0; k < D; ++k)
                d += oracle_bf16_to_f64(q[(size_t)h * D + k]) *
                     oracle_bf16_to_f64(K[(size_t)t * D + k]);
            sc[t] = scale * d;
            if (sc[t] > m) m = sc[t];
            any = 1;
        }
        for (int k = 0; k < D; ++k) {
            out[(size_t)h * D + k] = any ? 0.0 : NAN;
            if (absout) absout[(size_t)h * D + k] = any ? 0.0 : NAN;
        }
        if (!any) continue;
        double l = 0.0;
        for (int t = 0; t < T; ++t) {
            if (sc[t] == -INFINITY) continue;
            const double p = exp(sc[t] - m);
            l += p;
            for (int k = 0; k < D; ++k) {
                const double v = oracle_bf16_to_f64(V[(size_t)t * D + k]);
                out[(size_t)h * D + k] += p * v;
                if (absout) absout[(size_t)h * D + k] += p * fabs(v);
            }
        }
        for (int k = 0; k < D; ++k) {
            out[(size_t)h * D + k] /= l;
            if (absout) absout[(size_t)h * D + k] /= l;
        }
    }
    free(sc);
}

/*
 * Per-row symmetric int8: each of the N rows of the fp32 matrix W (rows ldw
 * apart) is optionally rotated (block > 0: the same fp32 butterfly FWHT per
 * block as oracle_quantize), then a = max |v| (fp32), s = a / 127 (fp32
 * division), q = s == 0 ? 0 : clamp(rint(v / s), -127, 127).  Q is [N][K]
 * int8, S[N] the fp32 scales.
 */
void oracle_quantize_rows_i8(const float* W, int N, int K, int ldw, int block, int8_t* Q,
                             float* S)
{
    float* v = (float*)malloc(sizeof(float) * (size_t)K);
    const float norm = block ? (float)(1.0 / sqrt((double)block)) : 1.0f;
    for (int n = 0; n < N; ++n) {
        for (int k = 0; k < K; ++k) v[k] = W[(size_t)n * ldw + k];
        if (block) {
            for (int b0 = 0; b0 < K; b0 += block) {
                float* x = v + b0;
                for (int h = 1; h < block; h *= 2)
                    for (int i = 0; i < block; i += 2 * h)
                        for (int j = i; j < i + h; ++j) {
                            const float a = x[j], b = x[j + h];
                            x[j] = a + b;
                            x[j + h] = a - b;
                        }
                for (int j = 0; j < block; ++j) x[j] = x[j] * norm;
            }
        }
        float a = 0.0f;
        for (int k = 0; k < K; ++k)
            if (fabsf(v[k]) > a) a = fabsf(v[k]);
        const float sc = a / 127.0f;
        S[n] = sc;
        for (int k = 0; k < K; ++k) {
            float q = 0.0f;
            if (sc != 0.0f) {
                q = rintf(v[k] / sc);
                if (q < -127.0f) q = -127.0f;
                if (q > 127.0f) q = 127.0f;
            }
            Q[(size_t)n * K + k] = (int8_t)q;
        }
    }
    free(v);
}

/*
 * Y[m][n] = (sum_k Xq[m][k] * Wq[n][k]) * xs[m] * ws[n]: the integer sum is
 * exact (64-bit), the scaling fp64.
 */
void oracle_gemm_i8(const int8_t* Xq, const float* xs, const int8_t* Wq, const float* ws,
                    int M, int N, int K, double* Y)
{
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            long long acc = 0;
            for (int k = 0; k < K; ++k)
                acc += (long long)Xq[(size_t)m * K + k] * (long long)Wq[(size_t)n * K + k];
            Y[(size_t)m * N + n] = (double)acc * (double)xs[m] * (double)ws[n];
        }
}
