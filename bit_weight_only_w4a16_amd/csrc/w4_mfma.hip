// w4_mfma.hip -- prefill-shaped W4A16 GEMM on the matrix cores.
//
// [P2] "fastgemma -- Gemma 4 E2B, CPU-only, AMX INT8 / AVX-512 VNNI":
// section "Why AMX for GEMM but not for attention" -- a weight GEMM reuses
// each weight byte across all M activation rows, so at prefill row counts it
// is bound by the multiply units, not memory; section "What is in the file" --
// int4 weights in groups of 256, rotated along K (the activations get a
// run-time Walsh-Hadamard transform before this kernel).  [P1] "Gemma 4 E2B on
// a 4 GB GPU with plain PyTorch, faster than llama.cpp" unpacks each layer to
// a full matrix before its GEMM (paragraph on prompt reads); this kernel never
// writes a dequantized matrix.
//
// v_mfma_f32_16x16x32_bf16 (A 16x32, B 32x16, D 16x16; lane l holds
// A[l%16][8(l/16) + j], B[8(l/16) + j][l%16] for j = 0..7, and
// D[4(l/16) + r][l%16] for r = 0..3).  B is W^T: lane l's eight B values are
// eight consecutive codes of weight row n = l%16, which is one device word,
// decoded with one shift and one and-or per pair to exact bf16 integers
// 128 + c.  Per K-group, the products accumulate from zero; the group's result
// is scale * (acc - acc136), where acc136 is the same MFMA against a B made of
// the bf16 value 136 (the decode bias plus the code offset 8): a column whose
// codes are all 8 goes through the identical arithmetic and cancels exactly.
//
// Tiling: each wave computes a (16 MF) x (16 NF) block of Y with no LDS and no
// barrier; the four waves of a workgroup take four consecutive M blocks of the
// same N block, so the weight words they load are shared through L1/L2, and
// workgroups with the same N block are numbered 8 apart so that, with the
// round-robin placement of workgroups on the 8 XCDs, they share an L2.
// Group 256 (rotated prefill format): one "super-step" covers 128 K; lane l
// loads 16 bytes of codes (four words) of its row and, in MFMA step s, uses
// word s for K = 32(l/16) + 8s + j -- the same permutation of K on both
// operands, which a dot product allows.  Group 32: one step of 32 K per group.
#include <cstdio>

#include "w4_dispatch.h"

namespace w4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct MfmaArgs {
    const uint32_t* codes;   // N x K/8 device words
    const uint16_t* scales;  // N x G bf16
    const uint16_t* X;       // M x K bf16, row stride ldx
    void* Y;                 // M x N, row stride ldy
    int M, N, K, G, group, ldx, ldy, ydt;
    int m_groups;            // workgroups per N block (4 M blocks each)
    int n_blocks;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 decode_word(uint32_t w, const DecodeConsts& k) {
    return u32x4{decode_pair(w, 0, k), decode_pair(w, 1, k), decode_pair(w, 2, k),
                 decode_pair(w, 3, k)};
}

template <int MF, int NF, bool SUPER>
__global__ __launch_bounds__(256) void mfma_gemm_kernel(MfmaArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15, lk = lane >> 4;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int nb = (slot / a.m_groups) * 8 + xcd;
    const int mg = slot % a.m_groups;
    if (nb >= a.n_blocks) return;
    const int mb = mg * 4 + wave;
    const int m0 = mb * 16 * MF, n0 = nb * 16 * NF;
    if (m0 >= a.M) return;
    const DecodeConsts k = decode_consts();
    const u32x4 b136 = {kOffsetPair, kOffsetPair, kOffsetPair, kOffsetPair};
    const int KW = a.K / 8;

    // rows past M / N are clamped to valid memory and never stored
    const uint16_t* xrow[MF];
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
        int m = m0 + 16 * mf + li;
        m = m < a.M ? m : a.M - 1;
        xrow[mf] = a.X + (size_t)m * a.ldx;
    }
    const uint32_t* crow[NF];
    const uint16_t* srow[NF];
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) {
        int n = n0 + 16 * nf + li;
        n = n < a.N ? n : a.N - 1;
        crow[nf] = a.codes + (size_t)n * KW;
        srow[nf] = a.scales + (size_t)n * a.G;
    }

    f32x4 tot[MF][NF];
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) tot[mf][nf] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int g = 0; g < a.G; ++g) {
        f32x4 acc[MF][NF], a136[MF];
#pragma unroll
        for (int mf = 0; mf < MF; ++mf) {
            a136[mf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int nf = 0; nf < NF; ++nf) acc[mf][nf] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (SUPER) {
            for (int kb = g * a.group; kb < (g + 1) * a.group; kb += 128) {
                u32x4 w[NF];
#pragma unroll
                for (int nf = 0; nf < NF; ++nf)
                    w[nf] = *reinterpret_cast<const u32x4*>(crow[nf] + kb / 8 + 4 * lk);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    u32x4 xa[MF];
#pragma unroll
                    for (int mf = 0; mf < MF; ++mf)
                        xa[mf] = *reinterpret_cast<const u32x4*>(xrow[mf] + kb + 32 * lk + 8 * s);
#pragma unroll
                    for (int nf = 0; nf < NF; ++nf) {
                        const u32x4 bv = decode_word(w[nf][s], k);
#pragma unroll
                        for (int mf = 0; mf < MF; ++mf) acc[mf][nf] = mfma(xa[mf], bv, acc[mf][nf]);
                    }
#pragma unroll
                    for (int mf = 0; mf < MF; ++mf) a136[mf] = mfma(xa[mf], b136, a136[mf]);
                }
            }
        } else {
            const int k0 = g * 32;  // group 32: one step
            u32x4 xa[MF];
#pragma unroll
            for (int mf = 0; mf < MF; ++mf)
                xa[mf] = *reinterpret_cast<const u32x4*>(xrow[mf] + k0 + 8 * lk);
#pragma unroll
            for (int nf = 0; nf < NF; ++nf) {
                const u32x4 bv = decode_word(crow[nf][k0 / 8 + lk], k);
#pragma unroll
                for (int mf = 0; mf < MF; ++mf) acc[mf][nf] = mfma(xa[mf], bv, acc[mf][nf]);
            }
#pragma unroll
            for (int mf = 0; mf < MF; ++mf) a136[mf] = mfma(xa[mf], b136, a136[mf]);
        }
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) {
            const float sc = bf16_to_f32(srow[nf][g]);
#pragma unroll
            for (int mf = 0; mf < MF; ++mf)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    tot[mf][nf][r] = fmaf(sc, acc[mf][nf][r] - a136[mf][r], tot[mf][nf][r]);
        }
    }

#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) {
            const int n = n0 + 16 * nf + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 16 * mf + 4 * lk + r;
                if (m < a.M && n < a.N) store_out(a.Y, (size_t)m * a.ldy + n, tot[mf][nf][r], a.ydt);
            }
        }
}

struct MfmaPlan {
    int MF, NF, m_blocks, n_blocks, m_groups, grid;
};

static MfmaPlan plan_mfma(int M, int N) {
    MfmaPlan p;
    p.MF = 4;
    p.NF = M <= 64 ? 2 : 4;  // short M: narrower N blocks for more workgroups
    p.m_blocks = (M + 16 * p.MF - 1) / (16 * p.MF);
    p.n_blocks = (N + 16 * p.NF - 1) / (16 * p.NF);
    p.m_groups = (p.m_blocks + 3) / 4;
    // workgroup b -> N block (b/8 / m_groups)*8 + b%8: round N blocks up to 8
    const int nb8 = (p.n_blocks + 7) / 8 * 8;
    p.grid = nb8 * p.m_groups;
    return p;
}

int launch_mfma_gemm(const void* packed, int N, int K, int group, int M, const uint16_t* X,
                     int ldx, void* Y, int ldy, int ydt, hipStream_t s) {
    const MfmaPlan p = plan_mfma(M, N);
    MfmaArgs a;
    a.codes = static_cast<const uint32_t*>(packed);
    a.scales = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(packed) +
                                                 scale_offset(N, K));
    a.X = X;
    a.Y = Y;
    a.M = M;
    a.N = N;
    a.K = K;
    a.group = group;
    a.G = K / group;
    a.ldx = ldx;
    a.ldy = ldy;
    a.ydt = ydt;
    a.m_groups = p.m_groups;
    a.n_blocks = p.n_blocks;
    const dim3 g(p.grid), b(256);
    const bool super = group % 128 == 0;
    if (p.NF == 2) {
        if (super)
            mfma_gemm_kernel<4, 2, true><<<g, b, 0, s>>>(a);
        else
            mfma_gemm_kernel<4, 2, false><<<g, b, 0, s>>>(a);
    } else {
        if (super)
            mfma_gemm_kernel<4, 4, true><<<g, b, 0, s>>>(a);
        else
            mfma_gemm_kernel<4, 4, false><<<g, b, 0, s>>>(a);
    }
    return hip_fail(hipGetLastError(), "gemm launch");
}

void describe_mfma(int M, int N, int K, int group, char* buf, size_t len) {
    const MfmaPlan p = plan_mfma(M, N);
    snprintf(buf, len, "mfma 16x16x32 wave tile %dx%d %s grid=%d (K=%d g=%d)", 16 * p.MF,
             16 * p.NF, group % 128 == 0 ? "super-step 128" : "step 32", p.grid, K, group);
}

}  // namespace w4
