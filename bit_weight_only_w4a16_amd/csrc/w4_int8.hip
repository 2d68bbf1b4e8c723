// w4_int8.hip -- the int8 twin: per-row int8 quantization and the int8 GEMM.
//
// [P2] "fastgemma -- Gemma 4 E2B, CPU-only, AMX INT8 / AVX-512 VNNI",
// section "What is in the file": every FFN weight is also stored as an int8
// twin (twice the int4 bytes), and prefill runs on int8, selected
// automatically at 16 rows or more (FGM_WEIGHTS=auto:16), decode on int4.
// Both operands of that product are int8; on MI355X the int8 matrix cores
// (v_mfma_i32_16x16x64_i8) run at twice the bf16 rate, which is the same
// reason to keep the twin.  Quantization rule (not on the page; the reading
// taken): each row -- of the rotated weight W', and at run time of the
// rotated activations x' -- gets its own fp32 scale s = max|v| / 127 and
// codes q = clamp(round_half_even(v / s), -127, 127); the product is the exact
// integer sum times both scales.
#include <cstdio>
#include <cstdlib>

#include "w4_config.h"
#include "w4_dispatch.h"
#include "w4_ring.h"

namespace w4 {

namespace {
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 mma_i8(u32x4 a, u32x4 b, i32x4 c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a),
                                                 __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}
}  // namespace

// One workgroup (4 waves) per row; wave w takes the row's 512-element spans
// w, w + 4, ... (lane l holds elements 8l .. 8l+7 of a span).  The spans are
// rotated once (the butterfly FWHT of w4_quantize: spans 1, 2, 4 inside a
// lane, 8 .. block/2 across lanes, then one fp32 scaling) and kept in
// registers for rows of up to 4 * kQMaxSpans spans (recomputed, identically,
// beyond); max |v| is reduced across the lanes and, through LDS, across the
// waves; then the codes are written.
constexpr int kQMaxSpans = 4;

template <bool BF16IN>
__global__ __launch_bounds__(256) void quant_rows_i8_kernel(const void* __restrict__ W, int ldw,
                                                           int N, int K, int block, float hscale,
                                                           int8_t* __restrict__ Q, int ldq,
                                                           float* __restrict__ S) {
    __shared__ float wmax[4];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = blockIdx.x;
    const int spans = (K + 511) / 512;

    auto span_vals = [&](int sp, float (&v)[8]) {
        const int k0 = sp * 512 + 8 * lane;
        if (k0 < K) {
            if (BF16IN) {
                const u32x4 w = gload(reinterpret_cast<const u32x4*>(
                    static_cast<const uint16_t*>(W) + (size_t)row * ldw + k0));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[2 * i] = __uint_as_float(w[i] << 16);
                    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
                }
            } else {
                const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(W) +
                                                                (size_t)row * ldw + k0);
                const u32x4 a = gload(p), b = gload(p + 1);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[i] = __uint_as_float(a[i]);
                    v[4 + i] = __uint_as_float(b[i]);
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = 0.f;
        }
        if (block) {
#pragma unroll
            for (int h = 1; h < 8; h *= 2) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if ((e & h) == 0) {
                        const float a = v[e], c = v[e + h];
                        v[e] = a + c;
                        v[e + h] = a - c;
                    }
                }
            }
            for (int d = 1; d < block / 8; d *= 2) {
                const bool upper = (lane & d) != 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float o = __shfl_xor(v[e], d, 64);
                    v[e] = upper ? (o - v[e]) : (v[e] + o);
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = v[e] * hscale;
        }
    };

    float cache[kQMaxSpans][8];
    float amax = 0.f;
    for (int i = 0, sp = wave; sp < spans; ++i, sp += 4) {
        float v[8];
        span_vals(sp, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
#pragma unroll
        for (int c = 0; c < kQMaxSpans; ++c)
            if (c == i)
#pragma unroll
                for (int e = 0; e < 8; ++e) cache[c][e] = v[e];
    }
    for (int d = 1; d < 64; d *= 2) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
    if (lane == 0) wmax[wave] = amax;
    __syncthreads();
    const float rmax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float sc = rmax / 127.f;
    if (threadIdx.x == 0) gstore(S + row, sc);

    for (int i = 0, sp = wave; sp < spans; ++i, sp += 4) {
        float v[8];
        if (i < kQMaxSpans) {
#pragma unroll
            for (int c = 0; c < kQMaxSpans; ++c)
                if (c == i)
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = cache[c][e];
        } else {
            span_vals(sp, v);
        }
        uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float q = 0.f;
            if (sc != 0.f) q = fminf(fmaxf(__builtin_rintf(v[e] / sc), -127.f), 127.f);
            const uint32_t b = (uint32_t)(int)q & 0xFFu;
            if (e < 4)
                w0 |= b << (8 * e);
            else
                w1 |= b << (8 * (e - 4));
        }
        const int k0 = sp * 512 + 8 * lane;
        if (k0 < K) {
            uint32_t* dst = reinterpret_cast<uint32_t*>(Q + (size_t)row * ldq + k0);
            gstore(dst, w0);
            gstore(dst + 1, w1);
        }
    }
}

int launch_quantize_rows_i8(const void* W, int wdt, int ldw, int N, int K, int block, int8_t* Q,
                            int ldq, float* S, hipStream_t s) {
    const float hscale = block ? (float)(1.0 / __builtin_sqrt((double)block)) : 1.f;
    const dim3 g((unsigned)N), b(256);
    if (wdt == W4_BF16)
        quant_rows_i8_kernel<true><<<g, b, 0, s>>>(W, ldw, N, K, block, hscale, Q, ldq, S);
    else
        quant_rows_i8_kernel<false><<<g, b, 0, s>>>(W, ldw, N, K, block, hscale, Q, ldq, S);
    return hip_fail(hipGetLastError(), "int8 quantize launch");
}

// ---------------------------------------------------------------- GEMM ---
//
// Y[m][n] = (sum_k Xq[m][k] Wq[n][k]) * xs[m] * ws[n], on v_mfma_i32_16x16x64_i8
// (A 16x64, B 64x16, D 16x16; lane l holds A[l%16][16(l/16) + j] and
// B[16(l/16) + j][l%16] for j = 0..15, and D[4(l/16) + r][l%16] for r = 0..3,
// checked on the hardware).  B is W^T, so a lane's B bytes are 16 consecutive
// codes of weight row n = l%16, like its A bytes of activation row l%16.
// A 256-thread workgroup (2 x 2 waves) computes a BM x BN block; K advances in
// 128-wide stages copied into padded LDS rows, the next stage's tiles in
// flight in registers while the current one is multiplied (one barrier per
// stage).  Blocks are numbered so that all M blocks of an N block run on one
// XCD, which then reads those weight rows once.
constexpr int kI8StageK = 128;
constexpr int kI8Row = kI8StageK + 16;  // LDS bytes per row (padded)

struct I8Args {
    const int8_t* X;
    const float* xs;
    const int8_t* W;
    const float* ws;
    void* Y;
    int M, N, K, ldx, ldw, ldy, ydt, m_blocks, n_blocks;
    int vec_out;  // Y and its row stride allow 16-byte stores
};

template <int MF, int NF>
__global__ __launch_bounds__(256) void gemm_i8_kernel(I8Args a) {
    constexpr int WN = 2;
    constexpr int BM = 2 * MF * 16, BN = WN * NF * 16;
    constexpr int CPR = kI8StageK / 16;  // 16-byte chunks per row and stage
    constexpr int A_CHUNKS = BM * CPR / 256, B_CHUNKS = BN * CPR / 256;
    static_assert(A_CHUNKS * 256 == BM * CPR && B_CHUNKS * 256 == BN * CPR, "tile split");
    __shared__ __align__(16) int8_t As[2][BM * kI8Row];
    __shared__ __align__(16) int8_t Bs[2][BN * kI8Row];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lk = lane >> 4;
    const int wm = wave / WN, wn = wave % WN;
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int mb = j % a.m_blocks;
    const int nb = (j / a.m_blocks) * 8 + xcd;
    if (nb >= a.n_blocks) return;
    const int m0 = mb * BM, n0 = nb * BN;
    const int stages = a.K / kI8StageK;

    // this thread's share of each stage's tiles (rows past M / N clamped to
    // valid memory and never stored)
    const int8_t* asrc[A_CHUNKS];
    int aoff[A_CHUNKS];
#pragma unroll
    for (int c = 0; c < A_CHUNKS; ++c) {
        const int idx = tid + 256 * c, r = idx / CPR, q = idx % CPR;
        const int m = m0 + r < a.M ? m0 + r : a.M - 1;
        asrc[c] = a.X + (size_t)m * a.ldx + 16 * q;
        aoff[c] = r * kI8Row + 16 * q;
    }
    const int8_t* bsrc[B_CHUNKS];
    int boff[B_CHUNKS];
#pragma unroll
    for (int c = 0; c < B_CHUNKS; ++c) {
        const int idx = tid + 256 * c, r = idx / CPR, q = idx % CPR;
        const int n = n0 + r < a.N ? n0 + r : a.N - 1;
        bsrc[c] = a.W + (size_t)n * a.ldw + 16 * q;
        boff[c] = r * kI8Row + 16 * q;
    }
    u32x4 ra[A_CHUNKS], rb[B_CHUNKS];
    auto fetch = [&](int st) {
#pragma unroll
        for (int c = 0; c < A_CHUNKS; ++c)
            ra[c] = gload(reinterpret_cast<const u32x4*>(asrc[c] + (size_t)st * kI8StageK));
#pragma unroll
        for (int c = 0; c < B_CHUNKS; ++c)
            rb[c] = nt_load(reinterpret_cast<const u32x4*>(bsrc[c] + (size_t)st * kI8StageK));
    };
    auto put = [&](int buf) {
#pragma unroll
        for (int c = 0; c < A_CHUNKS; ++c) *reinterpret_cast<u32x4*>(&As[buf][aoff[c]]) = ra[c];
#pragma unroll
        for (int c = 0; c < B_CHUNKS; ++c) *reinterpret_cast<u32x4*>(&Bs[buf][boff[c]]) = rb[c];
    };

    i32x4 acc[MF][NF];
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) acc[mf][nf] = i32x4{0, 0, 0, 0};

    const int arow0 = (wm * MF * 16 + li) * kI8Row + 16 * lk;
    const int brow0 = (wn * NF * 16 + li) * kI8Row + 16 * lk;
    fetch(0);
    put(0);
    __syncthreads();
    for (int st = 0; st < stages; ++st) {
        const int buf = st & 1;
        if (st + 1 < stages) fetch(st + 1);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            u32x4 xa[MF], wb[NF];
#pragma unroll
            for (int mf = 0; mf < MF; ++mf)
                xa[mf] = *reinterpret_cast<const u32x4*>(&As[buf][arow0 + mf * 16 * kI8Row + 64 * t]);
#pragma unroll
            for (int nf = 0; nf < NF; ++nf)
                wb[nf] = *reinterpret_cast<const u32x4*>(&Bs[buf][brow0 + nf * 16 * kI8Row + 64 * t]);
#pragma unroll
            for (int mf = 0; mf < MF; ++mf)
#pragma unroll
                for (int nf = 0; nf < NF; ++nf) acc[mf][nf] = mma_i8(xa[mf], wb[nf], acc[mf][nf]);
        }
        if (st + 1 < stages) {
            // buffer buf ^ 1 was last read in stage st - 1, which every wave
            // finished before the previous barrier
            put(buf ^ 1);
            __syncthreads();
        }
    }

#pragma unroll
    for (int nf = 0; nf < NF; ++nf) {
        const int n = n0 + wn * NF * 16 + 16 * nf + li;
        const float wsn = gload(a.ws + (n < a.N ? n : a.N - 1));
#pragma unroll
        for (int mf = 0; mf < MF; ++mf)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * MF * 16 + 16 * mf + 4 * lk + r;
                if (m < a.M && n < a.N) {
                    const float y = ((float)acc[mf][nf][r] * gload(a.xs + m)) * wsn;
                    store_out(a.Y, (size_t)m * a.ldy + n, y, a.ydt);
                }
            }
    }
}

// DMA-ring int8 GEMM (the layout and pipeline of the int4 prefill ring in
// w4_prefill.hip, without the decode).  Four waves side by side
// along N share one 64-row activation tile; each wave owns 16*NF weight rows
// and computes 64 x 16*NF outputs.  64-wide K stages (one MFMA step) are
// DMA'd into an LDS ring of SLOTS slots, P stages per wait and barrier.  Rows
// are 64 bytes per slot; position p of row r holds 16-byte chunk
// p ^ swz_i8(r), which keeps every fragment read free of bank
// conflicts on 32- and 64-bank LDS.  Scales are applied once, at the end,
// in the order of the register-staged kernel: (acc * xs[m]) * ws[n].
constexpr int kI8RingStage = 64;
constexpr int kI8RingRow = 64;   // bytes of a row in a slot

// r is any row index; only its place within its 16-row fragment counts,
// which is what the fragment reads see
__device__ __forceinline__ int swz_i8(int r) { return (((r & 15) >> 1) ^ ((r & 15) >> 3)) & 3; }

template <int NF, int SLOTS, int P, int KS>
__global__ __launch_bounds__(256 * KS) __attribute__((amdgpu_waves_per_eu(KS > 2 ? KS : 2)))
void gemm_i8_ring_kernel(I8Args a) {
    using namespace ring;
    constexpr int MF = 4, BM = 64, WN = 16 * NF, BN = 4 * WN;
    constexpr int A_BYTES = BM * kI8RingRow;          // one 16-byte DMA per wave
    constexpr int SLOT = A_BYTES + BN * kI8RingRow;   // + NF per wave
    constexpr int LOADS = 1 + NF;
    constexpr int OUT_ROW = BN * 4 + 16;
    constexpr int PART = 4 * 64 * MF * NF * 16;       // one K group's partial block
    static_assert(A_BYTES == 4 * 1024, "activation tile: one DMA per wave");
    static_assert(BM * OUT_ROW <= SLOTS * SLOT, "output staging fits in the ring");
    static_assert(KS == 1 || PART <= SLOTS * SLOT, "partial block fits in the group's ring");
    static_assert((P == 1 || P == 2) && SLOTS % P == 0 && SLOTS >= 2 * P, "ring of whole steps");
    static_assert(LOADS * (SLOTS - 2 * P) < 64, "vmcnt range");
    __shared__ __align__(16) uint8_t rings[KS * SLOTS * SLOT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave = wave_id & 3;   // position along N within the K group
    const int kg = wave_id >> 2;    // K group: a contiguous 1/KS of K
    uint8_t* const ring = rings + kg * (SLOTS * SLOT);
    const int li = lane & 15, lk = lane >> 4;
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int mb = j % a.m_blocks;
    const int nb = (j / a.m_blocks) * 8 + xcd;
    if (nb >= a.n_blocks) return;
    const int m0 = mb * BM, n0 = nb * BN;
    const int nw0 = n0 + wave * WN;
    const int stages = a.K / kI8RingStage / KS;   // this K group's stages
    const int kq = kg * stages * kI8RingStage;     // and its first K

    // scales of this lane's outputs, loaded now, used at the end
    float xsr[MF][4], wsr[NF];
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            xsr[mf][r] = gload(a.xs + min(m0 + 16 * mf + 4 * lk + r, a.M - 1));
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) wsr[nf] = gload(a.ws + min(nw0 + 16 * nf + li, a.N - 1));

    // DMA: lane l of an instruction fills row (l / 4), position (l & 3) of the
    // instruction's 16 rows; rows past M / N clamp to valid memory
    uint32_t aoff, boffs[NF];
    {
        const int r = 16 * wave + (lane >> 2);
        const int q = (lane & 3) ^ swz_i8(r);
        aoff = (uint32_t)((size_t)min(m0 + r, a.M - 1) * a.ldx + 16 * q);
    }
#pragma unroll
    for (int d = 0; d < NF; ++d) {
        const int iw = 16 * d + (lane >> 2);
        const int q = (lane & 3) ^ swz_i8(iw);
        boffs[d] = (uint32_t)((size_t)min(nw0 + iw, a.N - 1) * a.ldw + 16 * q);
    }
    const uint32_t ring0 = lds_addr(ring);
    const uint32_t adst = ring0 + 1024 * wave;
    const uint32_t bdst = ring0 + A_BYTES + wave * WN * kI8RingRow;
    auto issue = [&](int st, int slot) {
        const int8_t* ab = a.X + (size_t)(kq + st * kI8RingStage);
        const int8_t* bb = a.W + (size_t)(kq + st * kI8RingStage);
        dma16(aoff, ab, adst + slot * SLOT);
#pragma unroll
        for (int d = 0; d < NF; ++d) dma16(boffs[d], bb, bdst + slot * SLOT + 1024 * d);
    };

    const int sl = swz_i8(li);
    const int aread = li * kI8RingRow + 16 * (lk ^ sl);
    const int bread = A_BYTES + (wave * WN + li) * kI8RingRow + 16 * (lk ^ sl);
    i32x4 acc[MF][NF];
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) acc[mf][nf] = i32x4{0, 0, 0, 0};

    auto compute = [&](auto slc) {
        constexpr int SL = decltype(slc)::value;
        const uint8_t* slot = ring + SL * SLOT;
        u32x4 xa[MF], wb[NF];
#pragma unroll
        for (int mf = 0; mf < MF; ++mf)
            xa[mf] = *reinterpret_cast<const u32x4*>(slot + aread + mf * 16 * kI8RingRow);
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
            wb[nf] = *reinterpret_cast<const u32x4*>(slot + bread + nf * 16 * kI8RingRow);
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
#pragma unroll
            for (int mf = 0; mf < MF; ++mf) acc[mf][nf] = mma_i8(xa[mf], wb[nf], acc[mf][nf]);
    };
    auto step = [&](int s0, auto slc) {
        constexpr int SL0 = decltype(slc)::value * P;
        // stages issued after s0 + P - 1 by this wave
        wait_stage<LOADS, SLOTS - 2 * P>(stages - P - s0);
        // every wave's DMA of these stages has landed, and every wave has
        // finished the previous P stages, whose slots the next issue refills
        ring_barrier();
        static_for<P>([&](auto ic) {
            constexpr int I = decltype(ic)::value;
            if (s0 + SLOTS - P + I < stages)
                issue(s0 + SLOTS - P + I, (SL0 + SLOTS - P + I) % SLOTS);
        });
        static_for<P>([&](auto ic) { compute(std::integral_constant<int, SL0 + decltype(ic)::value>{}); });
    };

    const int pro = stages < SLOTS - P ? stages : SLOTS - P;
    for (int st = 0; st < pro; ++st) issue(st, st);
    // stage st lives in slot st % SLOTS (stages is a multiple of 2, so of P)
    for (int st0 = 0; st0 < stages; st0 += SLOTS)
        static_for<SLOTS / P>([&](auto slc) {
            const int s0 = st0 + P * decltype(slc)::value;
            if (s0 < stages) step(s0, slc);
        });

    // every DMA was waited for in the last step: after this barrier the ring
    // holds the output tile, which then leaves as whole 16-byte row pieces
    ring_barrier();
    // K groups 1 .. KS - 1 leave their integer partials in their own rings and
    // K group 0 adds them: integer sums, so the result is bitwise that of one
    // group walking all of K
    if (KS > 1) {
        if (kg > 0) {
            i32x4* part = reinterpret_cast<i32x4*>(ring) + (wave * MF * NF) * 64 + lane;
#pragma unroll
            for (int mf = 0; mf < MF; ++mf)
#pragma unroll
                for (int nf = 0; nf < NF; ++nf) part[(mf * NF + nf) * 64] = acc[mf][nf];
        }
        __syncthreads();
        if (kg == 0) {
#pragma unroll
            for (int q = 1; q < KS; ++q) {
                const i32x4* part = reinterpret_cast<const i32x4*>(rings + q * (SLOTS * SLOT)) +
                                    (wave * MF * NF) * 64 + lane;
#pragma unroll
                for (int mf = 0; mf < MF; ++mf)
#pragma unroll
                    for (int nf = 0; nf < NF; ++nf) acc[mf][nf] += part[(mf * NF + nf) * 64];
            }
        }
    }
    const bool f32 = a.ydt == W4_F32;
    const int esz = f32 ? 4 : 2;
    uint8_t* const ostage = rings;   // K group 0's ring
    if (kg == 0) {
#pragma unroll
        for (int mf = 0; mf < MF; ++mf)
#pragma unroll
            for (int nf = 0; nf < NF; ++nf)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float y = ((float)acc[mf][nf][r] * xsr[mf][r]) * wsr[nf];
                    uint8_t* p = ostage + (16 * mf + 4 * lk + r) * OUT_ROW +
                                 (wave * WN + 16 * nf + li) * esz;
                    if (f32)
                        *reinterpret_cast<float*>(p) = y;
                    else
                        *reinterpret_cast<uint16_t*>(p) = (uint16_t)f32_to_bf16_rne(y);
                }
    }
    __syncthreads();
    const int per = 16 / esz;
    const int cpr = BN / per;
    for (int e = tid; e < BM * cpr; e += 256 * KS) {
        const int row = e / cpr, c = e - row * cpr;
        const int m = m0 + row;
        if (m >= a.M) break;
        const int n = n0 + c * per;
        if (n >= a.N) continue;
        const u32x4 v = *reinterpret_cast<const u32x4*>(ostage + row * OUT_ROW + 16 * c);
        uint8_t* dst = static_cast<uint8_t*>(a.Y) + ((size_t)m * a.ldy + n) * esz;
        if (a.vec_out && n + per <= a.N) {
            gstore(reinterpret_cast<u32x4*>(dst), v);
        } else {
            for (int i = 0; i < per && n + i < a.N; ++i) {
                if (f32)
                    gstore(reinterpret_cast<uint32_t*>(dst) + i, v[i]);
                else
                    gstore(reinterpret_cast<uint16_t*>(dst) + i, (uint16_t)(v[i >> 1] >> (16 * (i & 1))));
            }
        }
    }
}

struct I8Plan {
    bool ring;                  // DMA-ring kernel (else register-staged)
    int cfg;                    // ring: index into kI8RingCfgs
    int MF, NF, BM, BN, m_blocks, n_blocks, grid;
};

struct I8RingCfg {
    int NF, slots, per_barrier, ks;
};
// 64 x 192 blocks for M > 256, 64 x 64 blocks (three times the workgroups)
// up to 256 rows, both with two 64-K stages per barrier (measured at N = 12288,
// K = 1536: 64 x 64 wins through M = 256, 64 x 192 from 512 on); entries 2
// and 3 split K over three or two wave groups, for 64 x 64 blocks that leave
// CUs idle
constexpr I8RingCfg kI8RingCfgs[] = {{3, 4, 2, 1}, {1, 6, 2, 1}, {1, 4, 2, 3}, {1, 6, 2, 2}};
constexpr int kI8NumRingCfgs = sizeof(kI8RingCfgs) / sizeof(kI8RingCfgs[0]);

static I8Plan plan_i8(int M, int N, int K, int ldx, int ldw) {
    I8Plan p;
    // W4_FORCE_PATH i8_regs selects the register-staged kernel (comparison
    // runs); W4_I8_RING=<cfg + 1> forces a ring configuration
    const auto c = config();
    // per-lane DMA offsets are 32-bit
    const bool fits = (size_t)(M - 1) * (size_t)ldx + (size_t)K < (1ull << 32) &&
                      (size_t)(N - 1) * (size_t)ldw + (size_t)K < (1ull << 32);
    p.ring = fits && !(c->force & kForceI8Regs);
    if (p.ring) {
        p.cfg = M <= 256 ? 1 : 0;
        // one 64-row block (N / 64 workgroups, at most one per CU): split K
        const int st = K / kI8RingStage;
        if (p.cfg == 1 && (N + 63) / 64 * ((M + 63) / 64) <= kNumCUs)
            p.cfg = st % 6 == 0 ? 2 : (st % 4 == 0 ? 3 : 1);
        if (c->i8_ring >= 1 && c->i8_ring <= kI8NumRingCfgs) p.cfg = c->i8_ring - 1;
        // each K group needs a whole number of two-stage steps
        if (st % (2 * kI8RingCfgs[p.cfg].ks) != 0) p.cfg = M <= 256 ? 1 : 0;
        p.MF = 4;
        p.NF = kI8RingCfgs[p.cfg].NF;
        p.BM = 64;
        p.BN = 64 * p.NF;
    } else {
        // register-staged: measured on MI355X at N = 12288, K = 1536, M = 64..512,
        // 64 x 64 blocks (four workgroups per CU) beat 64 x 128, 128 x 64 and 128 x 128
        p.cfg = 0;
        p.MF = 2;
        p.NF = 2;
        if (c->i8_mf) {  // W4_I8_TILE "MF,NF": tuning override (2 or 4 each)
            p.MF = c->i8_mf;
            p.NF = c->i8_nf;
        }
        p.BM = 2 * p.MF * 16;
        p.BN = 2 * p.NF * 16;
    }
    p.m_blocks = (M + p.BM - 1) / p.BM;
    p.n_blocks = (N + p.BN - 1) / p.BN;
    p.grid = 8 * p.m_blocks * ((p.n_blocks + 7) / 8);
    return p;
}

int launch_gemm_i8(const int8_t* X, int ldx, const float* xs, const int8_t* W, int ldw,
                   const float* ws, int M, int N, int K, void* Y, int ldy, int ydt,
                   hipStream_t s) {
    const I8Plan p = plan_i8(M, N, K, ldx, ldw);
    I8Args a;
    a.X = X;
    a.xs = xs;
    a.W = W;
    a.ws = ws;
    a.Y = Y;
    a.M = M;
    a.N = N;
    a.K = K;
    a.ldx = ldx;
    a.ldw = ldw;
    a.ldy = ldy;
    a.ydt = ydt;
    a.m_blocks = p.m_blocks;
    a.n_blocks = p.n_blocks;
    const size_t esz = ydt == W4_F32 ? 4 : 2;
    a.vec_out = (reinterpret_cast<uintptr_t>(Y) % 16 == 0) && ((size_t)ldy * esz) % 16 == 0;
    const dim3 g(p.grid), b(p.ring ? 256 * kI8RingCfgs[p.cfg].ks : 256);
    if (p.ring) {
        switch (p.cfg) {
            case 0: gemm_i8_ring_kernel<3, 4, 2, 1><<<g, b, 0, s>>>(a); break;
            case 1: gemm_i8_ring_kernel<1, 6, 2, 1><<<g, b, 0, s>>>(a); break;
            case 2: gemm_i8_ring_kernel<1, 4, 2, 3><<<g, b, 0, s>>>(a); break;
            default: gemm_i8_ring_kernel<1, 6, 2, 2><<<g, b, 0, s>>>(a); break;
        }
    } else if (p.MF == 2 && p.NF == 2) {
        gemm_i8_kernel<2, 2><<<g, b, 0, s>>>(a);
    } else if (p.MF == 2) {
        gemm_i8_kernel<2, 4><<<g, b, 0, s>>>(a);
    } else if (p.NF == 2) {
        gemm_i8_kernel<4, 2><<<g, b, 0, s>>>(a);
    } else {
        gemm_i8_kernel<4, 4><<<g, b, 0, s>>>(a);
    }
    return hip_fail(hipGetLastError(), "int8 gemm launch");
}

void describe_i8(int M, int N, int K, char* buf, size_t len) {
    const I8Plan p = plan_i8(M, N, K, K, K);
    if (p.ring)
        snprintf(buf, len,
                 "int8 mfma 16x16x64 dma-ring block %dx%d waves %dx4 slots %d stage 64 x%d "
                 "grid=%d (K=%d)",
                 p.BM, p.BN, kI8RingCfgs[p.cfg].ks, kI8RingCfgs[p.cfg].slots,
                 kI8RingCfgs[p.cfg].per_barrier, p.grid, K);
    else
        snprintf(buf, len, "int8 mfma 16x16x64 block %dx%d waves 2x2 stage 128 grid=%d (K=%d)",
                 p.BM, p.BN, p.grid, K);
}

}  // namespace w4
