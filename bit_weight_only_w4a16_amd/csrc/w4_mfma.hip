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
// decoded to the exact bf16 values 16 (c - 8) (w4_common.h).  Per K-group the
// products accumulate from zero; the group's result is (scale / 16) * acc.
//
// Block tiling: a 256-thread workgroup (2 x 2 waves) computes a BM x BN block
// of Y; each wave a (16 MF) x (16 NF) part of it.  K advances in 128-wide
// stages: the workgroup copies the stage's activation tile (BM x 128 bf16) and
// code tile (BN x 64 bytes) from global memory into padded LDS buffers, and
// while the waves multiply stage s out of one buffer, the loads of stage s+1
// are already in flight into registers (double buffering, one barrier per
// stage).  Group 256: lane l takes the four code words 4(l/16)..4(l/16)+3 of
// its row in the stage and in MFMA step t uses word t for K = 32(l/16) + 8t +
// j; the activations are read with the same K permutation, which a dot product
// allows.  Group 32: step t is group t of the stage in natural K order.
// Workgroups are numbered so that all M blocks of an N block run on one XCD
// (workgroups go round-robin to the 8 XCDs): each XCD reads its weight
// columns once and keeps the activations in its L2.
#include <cstdio>
#include <cstdlib>

#include "w4_config.h"
#include "w4_dispatch.h"

namespace w4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kStageK = 128;                 // K per stage
constexpr int kArow = kStageK * 2 + 16;      // LDS bytes per activation row (padded)
constexpr int kBrow = kStageK / 2 + 16;      // LDS bytes per code row (padded)

struct MfmaArgs {
    const uint32_t* codes;   // N x K/8 device words
    const uint16_t* scales;  // N x G bf16
    const uint16_t* X;       // M x K bf16, row stride ldx
    void* Y;                 // M x N, row stride ldy
    int M, N, K, G, group, ldx, ldy, ydt;
    int m_blocks, n_blocks;
};

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}


template <int WM, int WN, int MF, int NF, bool SUPER>
__global__ __launch_bounds__(256) void mfma_gemm_kernel(MfmaArgs a) {
    constexpr int BM = WM * MF * 16, BN = WN * NF * 16;
    constexpr int A_CHUNKS = BM * (kStageK * 2 / 16) / 256;  // 16-byte loads per thread
    constexpr int B_CHUNKS = BN * (kStageK / 2 / 16) / 256;
    static_assert(WM * WN == 4, "four waves");
    static_assert(A_CHUNKS * 256 == BM * kStageK * 2 / 16, "activation tile split");
    static_assert(B_CHUNKS * 256 == BN * kStageK / 2 / 16, "code tile split");
    __shared__ __align__(16) uint8_t As[2][BM * kArow];
    __shared__ __align__(16) uint8_t Bs[2][BN * kBrow];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lk = lane >> 4;
    const int wm = wave / WN, wn = wave % WN;

    // block numbering: XCD x = b % 8 runs every M block of N blocks x, x+8, ...
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int mb = j % a.m_blocks;
    const int nb = (j / a.m_blocks) * 8 + xcd;
    if (nb >= a.n_blocks) return;
    const int m0 = mb * BM, n0 = nb * BN;
    const int KW = a.K / 8;
    const int stages = a.K / kStageK;

    // global sources of this thread's share of each stage's tiles (rows past
    // M / N are clamped to valid memory and never stored)
    const uint8_t* asrc[A_CHUNKS];
    int aoff[A_CHUNKS];
#pragma unroll
    for (int c = 0; c < A_CHUNKS; ++c) {
        const int idx = tid + 256 * c;
        const int r = idx / (kStageK * 2 / 16), q = idx % (kStageK * 2 / 16);
        int m = m0 + r;
        m = m < a.M ? m : a.M - 1;
        asrc[c] = reinterpret_cast<const uint8_t*>(a.X + (size_t)m * a.ldx) + 16 * q;
        aoff[c] = r * kArow + 16 * q;
    }
    const uint8_t* bsrc[B_CHUNKS];
    int boff[B_CHUNKS];
#pragma unroll
    for (int c = 0; c < B_CHUNKS; ++c) {
        const int idx = tid + 256 * c;
        const int r = idx / (kStageK / 2 / 16), q = idx % (kStageK / 2 / 16);
        int n = n0 + r;
        n = n < a.N ? n : a.N - 1;
        bsrc[c] = reinterpret_cast<const uint8_t*>(a.codes + (size_t)n * KW) + 16 * q;
        boff[c] = r * kBrow + 16 * q;
    }
    const uint16_t* srow[NF];
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) {
        int n = n0 + wn * NF * 16 + 16 * nf + li;
        n = n < a.N ? n : a.N - 1;
        srow[nf] = a.scales + (size_t)n * a.G;
    }

    u32x4 ra[A_CHUNKS], rb[B_CHUNKS];
    auto fetch = [&](int st) {
#pragma unroll
        for (int c = 0; c < A_CHUNKS; ++c)
            ra[c] = *reinterpret_cast<const u32x4*>(asrc[c] + (size_t)st * kStageK * 2);
#pragma unroll
        for (int c = 0; c < B_CHUNKS; ++c)
            rb[c] = nt_load(reinterpret_cast<const u32x4*>(bsrc[c] + (size_t)st * kStageK / 2));
    };
    auto put = [&](int buf) {
#pragma unroll
        for (int c = 0; c < A_CHUNKS; ++c)
            *reinterpret_cast<u32x4*>(&As[buf][aoff[c]]) = ra[c];
#pragma unroll
        for (int c = 0; c < B_CHUNKS; ++c)
            *reinterpret_cast<u32x4*>(&Bs[buf][boff[c]]) = rb[c];
    };

    f32x4 tot[MF][NF], acc[MF][NF];
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) {
            tot[mf][nf] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc[mf][nf] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    // fold the finished group g into tot and restart its partials
    auto close_group = [&](int g) {
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) {
            const float sc = bf16_to_f32(srow[nf][g]) * 0.0625f;
#pragma unroll
            for (int mf = 0; mf < MF; ++mf) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    tot[mf][nf][r] = fmaf(sc, acc[mf][nf][r], tot[mf][nf][r]);
                acc[mf][nf] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };

    const int arow0 = (wm * MF * 16 + li) * kArow;
    const int brow0 = (wn * NF * 16 + li) * kBrow;

    fetch(0);
    put(0);
    __syncthreads();
    for (int st = 0; st < stages; ++st) {
        const int buf = st & 1;
        if (st + 1 < stages) fetch(st + 1);
        const uint8_t* A = As[buf];
        const uint8_t* B = Bs[buf];
        if (SUPER) {
            u32x4 wv[NF];
#pragma unroll
            for (int nf = 0; nf < NF; ++nf)
                wv[nf] = *reinterpret_cast<const u32x4*>(B + brow0 + nf * 16 * kBrow + 16 * lk);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                u32x4 xa[MF];
#pragma unroll
                for (int mf = 0; mf < MF; ++mf)
                    xa[mf] = *reinterpret_cast<const u32x4*>(A + arow0 + mf * 16 * kArow +
                                                             2 * (32 * lk + 8 * t));
#pragma unroll
                for (int nf = 0; nf < NF; ++nf) {
                    const u32x4 bv = decode_x16(wv[nf][t]);
#pragma unroll
                    for (int mf = 0; mf < MF; ++mf) acc[mf][nf] = mfma(xa[mf], bv, acc[mf][nf]);
                }
            }
            if (((st + 1) * kStageK) % a.group == 0) close_group((st * kStageK) / a.group);
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                u32x4 xa[MF];
#pragma unroll
                for (int mf = 0; mf < MF; ++mf)
                    xa[mf] = *reinterpret_cast<const u32x4*>(A + arow0 + mf * 16 * kArow +
                                                             2 * (32 * t + 8 * lk));
#pragma unroll
                for (int nf = 0; nf < NF; ++nf) {
                    const uint32_t w = *reinterpret_cast<const uint32_t*>(
                        B + brow0 + nf * 16 * kBrow + 4 * (4 * t + lk));
                    const u32x4 bv = decode_x16(w);
#pragma unroll
                    for (int mf = 0; mf < MF; ++mf) acc[mf][nf] = mfma(xa[mf], bv, acc[mf][nf]);
                }
                close_group(st * 4 + t);
            }
        }
        if (st + 1 < stages) {
            // buffer buf ^ 1 was last read in stage st - 1, which every wave
            // finished before the previous barrier
            put(buf ^ 1);
            __syncthreads();
        }
    }

#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) {
            const int n = n0 + wn * NF * 16 + 16 * nf + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * MF * 16 + 16 * mf + 4 * lk + r;
                if (m < a.M && n < a.N) store_out(a.Y, (size_t)m * a.ldy + n, tot[mf][nf][r], a.ydt);
            }
        }
}

// Block shapes (2 x 2 waves): BM x BN with per-wave MF x NF fragments.
struct MfmaCfg {
    int MF, NF;
};
static const MfmaCfg kMfmaCfgs[] = {{2, 2}, {4, 4}, {2, 4}, {4, 2}};

struct MfmaPlan {
    int cfg;  // index into kMfmaCfgs
    int BM, BN, m_blocks, n_blocks, grid;
};

static MfmaPlan plan_mfma(int M, int N) {
    MfmaPlan p;
    // measured on MI355X at N = 12288, K = 1536: 64 x 64 blocks for short M,
    // 64 x 128 blocks (two workgroups per CU) beyond
    p.cfg = M <= 128 ? 0 : 2;
    const int o = config()->mfma_cfg;  // W4_MFMA_CFG: tuning override 0..3
    if (o >= 0 && o <= 3) p.cfg = o;
    p.BM = 32 * kMfmaCfgs[p.cfg].MF;
    p.BN = 32 * kMfmaCfgs[p.cfg].NF;
    p.m_blocks = (M + p.BM - 1) / p.BM;
    p.n_blocks = (N + p.BN - 1) / p.BN;
    p.grid = 8 * p.m_blocks * ((p.n_blocks + 7) / 8);
    return p;
}

template <int WM, int WN, int MF, int NF>
static void launch_cfg(bool super, dim3 g, hipStream_t s, const MfmaArgs& a) {
    if (super)
        mfma_gemm_kernel<WM, WN, MF, NF, true><<<g, dim3(256), 0, s>>>(a);
    else
        mfma_gemm_kernel<WM, WN, MF, NF, false><<<g, dim3(256), 0, s>>>(a);
}

// W4_FORCE_PATH prefill_regs keeps every shape on the register-staged kernel
// below (A/B comparisons); otherwise the shapes the DMA ring serves take it.
static bool use_ring(int M, int N, int K, int group, int ldx) {
    if (config()->force & kForcePrefillRegs) return false;
    return prefill_supported(M, N, K, group, ldx);
}

int launch_mfma_gemm(const void* packed, int N, int K, int group, int M, const uint16_t* X,
                     int ldx, void* Y, int ldy, int ydt, hipStream_t s) {
    if (use_ring(M, N, K, group, ldx)) return launch_prefill(packed, N, K, group, M, X, ldx, Y, ldy, ydt, s);
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
    a.m_blocks = p.m_blocks;
    a.n_blocks = p.n_blocks;
    const bool super = group % kStageK == 0;
    switch (p.cfg) {
        case 0: launch_cfg<2, 2, 2, 2>(super, dim3(p.grid), s, a); break;
        case 1: launch_cfg<2, 2, 4, 4>(super, dim3(p.grid), s, a); break;
        case 2: launch_cfg<2, 2, 2, 4>(super, dim3(p.grid), s, a); break;
        default: launch_cfg<2, 2, 4, 2>(super, dim3(p.grid), s, a); break;
    }
    return hip_fail(hipGetLastError(), "gemm launch");
}

void describe_mfma(int M, int N, int K, int group, char* buf, size_t len) {
    if (use_ring(M, N, K, group, K)) return describe_prefill(M, N, K, group, buf, len);
    const MfmaPlan p = plan_mfma(M, N);
    snprintf(buf, len, "mfma 16x16x32 block %dx%d waves 2x2 %s grid=%d (K=%d g=%d)", p.BM, p.BN,
             group % kStageK == 0 ? "stage 128 permuted" : "stage 128 by group", p.grid, K, group);
}

}  // namespace w4
