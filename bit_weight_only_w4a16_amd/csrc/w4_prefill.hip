// w4_prefill.hip -- prefill-shaped W4A16 GEMM on the matrix cores, fed by an
// LDS ring that the global-to-LDS DMA loads fill several stages ahead.
//
// [P2] "fastgemma -- Gemma 4 E2B, CPU-only, AMX INT8 / AVX-512 VNNI":
// section "Why AMX for GEMM but not for attention" -- a weight GEMM reuses each
// weight byte across all M activation rows, so at prefill row counts the
// multiply units bound it; section "What is in the file" -- int4 weights in
// groups of 256 (or 512), rotated along K; group 32 too (the format of the
// decode-step weights), where every 32-wide MFMA step is one scale group and
// is scaled on its own.  Same product as w4_mfma.hip:
// Y[m][n] = sum_g s[n][g] * sum_{k in g} (c[n][k] - 8) * x[m][k], fp32
// accumulation, no dequantized matrix in memory.
//
// Arithmetic (v_mfma_f32_16x16x32_bf16; lane l holds A[l%16][8(l/16) + j],
// B[8(l/16) + j][l%16], D[4(l/16) + r][l%16]):
//   - a lane's eight B values are one device word of weight row l%16, decoded
//     to the exact bf16 values 16 (c - 8) (w4_common.h), so every product is
//     exact and a code of 8 contributes an exact zero;
//   - per K-group the products accumulate from zero; the group adds
//     (s / 16) * acc to the total;
//   - within a 64-wide K stage, lane group l/16 takes device words
//     2(l/16), 2(l/16)+1 of its row, word t in MFMA step t, and the activation
//     fragment is read with the same K permutation (a dot product allows it).
//
// Work split: a workgroup holds KS groups of four waves.  The four waves of a
// group sit side by side along N and share one 16*MF-row activation tile;
// each wave owns 16*NF weight rows and computes a (16 MF) x (16 NF) block of
// Y, so a decoded word feeds MF MFMAs.  With KS > 1 each group takes a
// contiguous 1/KS of K (whole scale groups) through a ring of its own, and
// the groups' partial blocks are added in LDS in group order at the end: the
// same weight and activation bytes per workgroup, KS times the waves to hide
// each stage's latency, and 1/KS of the stages per wave (few-row products,
// whose workgroups do not fill the chip).  The block shapes hold two or
// three workgroups per CU (LDS and registers), and the host counts launch
// rounds at each one's occupancy.  Workgroups are numbered so that every M block of an N block runs on
// one XCD (workgroups go round-robin to the 8 XCDs): the weights are read from
// HBM once per XCD and the activations stay in that XCD's L2.
//
// Memory pipeline: SLOTS ring slots of one 64-wide K stage each.  Every wave
// issues its share of a stage as DMA loads straight into LDS (16-byte loads
// for activations, 4-byte loads for codes), SLOTS - 1 stages ahead of the one
// it multiplies; one explicit vmcnt wait plus one barrier per stage make a
// stage visible, and the barrier also proves the slot being refilled was
// released by every wave.  The compiler does not track these loads, so every
// wait on them is written out here; no other global load runs in the loop.
// The scales of the workgroup's rows are copied to LDS once, up front.
//
// LDS layouts (XOR swizzles keep every LDS read free of bank conflicts, for
// 32- and 64-bank LDS alike; the DMA writes each instruction's 64 lanes to
// consecutive addresses, so the swizzle is applied to the global side):
//   activation row r: 128 bytes, 8 chunks of 8 bf16; position p holds chunk
//     p ^ g(r), g(r) = (r & 7) ^ ((r >> 3) & 1);
//   code row i: 32 bytes, 4 units of 2 words; position P holds unit
//     P ^ h(i), h(i) = ((i & 15) >> 2) & 3.
#include <cstdio>
#include <cstdlib>
#include <type_traits>
#include <utility>

#include "w4_config.h"
#include "w4_dispatch.h"
#include "w4_ring.h"

namespace w4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace {

using namespace ring;

constexpr int kStage = 64;     // K per ring slot
constexpr int kARow = 128;     // bytes of an activation row in a slot
constexpr int kBRow = 32;      // bytes of a code row in a slot
constexpr int kMaxG = 32;      // scale groups per row kept in LDS (K = 8192 at g256)
constexpr int kMaxG32 = 48;    // the same for group 32 (K = 1536)
constexpr int kMaxG32Split = 192;   // group 32 in K-split workgroups (K = 6144),
                                    // which hold one workgroup per CU anyway

struct PfArgs {
    const uint32_t* codes;   // N x K/8 device words
    const uint16_t* scales;  // N x G bf16
    const uint16_t* X;       // M x K bf16, row stride ldx
    void* Y;                 // M x N, row stride ldy
    int M, N, K, G, group, ldx, ldy, ydt;
    int m_blocks, n_blocks;
    int vec_out;             // Y and its row stride allow 16-byte stores
};

template <int MF, int NF, int SLOTS, int KS>
struct PfShape {
    static constexpr int BM = 16 * MF;                 // activation rows per workgroup
    static constexpr int WN = 16 * NF;                 // weight rows per wave
    static constexpr int BN = 4 * WN;                  // weight rows per workgroup
    static constexpr int A_BYTES = BM * kARow;
    static constexpr int B_BYTES = BN * kBRow;
    static constexpr int SLOT = A_BYTES + B_BYTES;
    static constexpr int A_DMA = A_BYTES / 1024 / 4;   // 16-byte DMA per wave per stage
    static constexpr int B_DMA = WN * kBRow / 256;     // 4-byte DMA per wave per stage
    static constexpr int LOADS = A_DMA + B_DMA;        // vector-memory ops per wave per stage
    static_assert(A_DMA * 4 * 1024 == A_BYTES, "activation tile: whole DMA rounds per wave");
    static_assert(B_DMA * 256 == WN * kBRow, "code tile: whole DMA rounds per wave");
    static_assert(LOADS * (SLOTS - 2) < 64, "vmcnt range");
    static constexpr int OUT_ROW = BN * 4 + 16;        // padded fp32 staging row (bytes)
    // the output block is staged in the ring whole, or in two halves of rows
    static constexpr int OUT_PARTS = BM * OUT_ROW <= SLOTS * SLOT ? 1 : 2;
    static_assert(BM / OUT_PARTS * OUT_ROW <= SLOTS * SLOT, "output staging fits in the ring");
    static_assert(MF % OUT_PARTS == 0, "whole fragments per staged part");
    static constexpr int PART = 4 * 64 * MF * NF * 16; // one K group's partial block (bytes)
    static_assert(KS == 1 || PART <= SLOTS * SLOT, "partial block fits in the group's ring");
    static constexpr int THREADS = 256 * KS;
};

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ int swz_a(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz_b(int i) { return ((i & 15) >> 2) & 3; }

// MF = 8 (128 activation rows per wave; groups of 64 or more, two stages per
// barrier): one wave per SIMD with the registers of two, each decoded code
// word feeding eight MFMAs instead of four (half the decode per MFMA), and
// the activation fragments of the next 32-wide step read while the current
// step's MFMAs run (compute_pair).
// Waves per SIMD the registers are sized for: KS for K splits of three or
// more groups; one for 128 x 48 per wave; three for 64 x 32 per wave on a
// three-slot ring (44-48 KB of LDS: three workgroups per CU); two otherwise.
template <int MF, int NF, int SLOTS, int P, int KS, bool G32>
__global__ __launch_bounds__(256 * KS)
__attribute__((amdgpu_waves_per_eu(KS > 2 ? KS : (MF * NF > 16 ? 1 : (MF * NF <= 8 && SLOTS == 3 ? 3 : 2)))))
void prefill_kernel(PfArgs a) {
    using S = PfShape<MF, NF, SLOTS, KS>;
    static_assert(P == 1 || P == 2, "stages per barrier");
    static_assert(SLOTS % P == 0 && SLOTS >= 2 * P, "ring of whole steps, double-buffered at least");
    __shared__ __align__(16) uint8_t rings[KS * SLOTS * S::SLOT];
    __shared__ __align__(16) uint16_t sc[S::BN * (G32 ? (KS > 1 ? kMaxG32Split : kMaxG32) : kMaxG)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave = wave_id & 3;   // position along N within the K group
    const int kg = wave_id >> 2;    // K group
    uint8_t* const ring = rings + kg * (SLOTS * S::SLOT);
    const int li = lane & 15, lk = lane >> 4;

    // XCD x = blockIdx % 8 runs every M block of N blocks x, x + 8, ...
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int mb = j % a.m_blocks;
    const int nb = (j / a.m_blocks) * 8 + xcd;
    if (nb >= a.n_blocks) return;
    const int m0 = mb * S::BM, n0 = nb * S::BN;
    const int nw0 = n0 + wave * S::WN;
    const int KW = a.K / 8;
    const int stages = a.K / kStage / KS;   // this K group's stages
    const int kq = kg * stages * kStage;    // this K group's first K
    const int g0 = kq / a.group;            // and its first scale group
    const int G = a.G / KS;                 // scale groups per K group

    // DMA sources: a wave-uniform base that advances one stage per slot plus a
    // fixed 32-bit per-lane byte offset (the host keeps every offset below
    // 2^32); destinations: fixed per wave, plus the slot
    uint32_t aoffs[S::A_DMA];
#pragma unroll
    for (int d = 0; d < S::A_DMA; ++d) {
        const int r = 8 * (wave * S::A_DMA + d) + (lane >> 3);
        const int q = (lane & 7) ^ swz_a(r);
        const int m = min(m0 + r, a.M - 1);
        aoffs[d] = (uint32_t)(((size_t)m * a.ldx + 8 * q) * 2);
    }
    uint32_t boffs[S::B_DMA];
#pragma unroll
    for (int d = 0; d < S::B_DMA; ++d) {
        const int iw = 8 * d + (lane >> 3);          // row within the wave's rows
        const int p = lane & 7;                       // word position within the row
        const int word = 2 * ((p >> 1) ^ swz_b(iw)) + (p & 1);
        const int n = min(nw0 + iw, a.N - 1);
        boffs[d] = (uint32_t)(((size_t)n * KW + word) * 4);
    }
    const uint32_t ring0 = lds_addr(ring);
    const uint32_t adst = ring0 + 1024 * (wave * S::A_DMA);
    const uint32_t bdst = ring0 + S::A_BYTES + wave * S::WN * kBRow;
    auto issue = [&](int st, int slot) {
        const uint8_t* ab =
            reinterpret_cast<const uint8_t*>(a.X) + (size_t)(kq + st * kStage) * 2;
        const uint8_t* bb =
            reinterpret_cast<const uint8_t*>(a.codes) + (size_t)(kq + st * kStage) / 2;
#pragma unroll
        for (int d = 0; d < S::A_DMA; ++d) dma16(aoffs[d], ab, adst + slot * S::SLOT + 1024 * d);
#pragma unroll
        for (int d = 0; d < S::B_DMA; ++d) dma4(boffs[d], bb, bdst + slot * S::SLOT + 256 * d);
    };

    // per-lane LDS read offsets within a slot
    // Groups of 64 or more: MFMA step t takes words 2j + t of the stage (lane
    // group j = lk), one 8-byte code read per stage.  Group 32: step t takes
    // words 4t + j, so that each step is exactly one scale group (two 4-byte
    // code reads; both layouts stay free of bank conflicts).
    const int gl = swz_a(li);
    const int aoff0 = li * kARow + 16 * ((G32 ? lk : 2 * lk) ^ gl);
    const int aoff1 = li * kARow + 16 * ((G32 ? 4 + lk : 2 * lk + 1) ^ gl);
    const int brow = S::A_BYTES + wave * S::WN * kBRow + li * kBRow;
    const int boff = brow + 8 * (lk ^ swz_b(li));
    const int boff0 = brow + 8 * ((lk >> 1) ^ swz_b(li)) + 4 * (lk & 1);        // word lk
    const int boff1 = brow + 8 * ((2 + (lk >> 1)) ^ swz_b(li)) + 4 * (lk & 1);  // word 4 + lk
    const uint16_t* scrow = sc + (wave * S::WN + li) * a.G + g0;

    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 tot[MF][NF], acc[MF][NF];
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) tot[mf][nf] = zero;

    // One stage's products out of ring slot SL.  The first stage of a group
    // starts its MFMA chains from a zero accumulator operand.
    auto compute = [&](auto slc, auto firstc, int st) {
        constexpr int SL = decltype(slc)::value;
        constexpr bool FIRST = decltype(firstc)::value;
        const uint8_t* slot = ring + SL * S::SLOT;
        if constexpr (G32) {
            // every MFMA step is one whole scale group: products start from
            // zero, and each group is scaled into the totals at once (step t
            // of stage st is group 2 st + t)
            __builtin_amdgcn_sched_barrier(0);
            uint32_t bw[2][NF], sw[NF];
#pragma unroll
            for (int nf = 0; nf < NF; ++nf) {
                bw[0][nf] = *reinterpret_cast<const uint32_t*>(slot + boff0 + nf * 16 * kBRow);
                bw[1][nf] = *reinterpret_cast<const uint32_t*>(slot + boff1 + nf * 16 * kBRow);
                sw[nf] = *reinterpret_cast<const uint32_t*>(scrow + nf * 16 * a.G + 2 * st);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                u32x4 xa[MF];
#pragma unroll
                for (int mf = 0; mf < MF; ++mf)
                    xa[mf] = *reinterpret_cast<const u32x4*>(slot + (t ? aoff1 : aoff0) +
                                                             mf * 16 * kARow);
#pragma unroll
                for (int nf = 0; nf < NF; ++nf) {
                    const u32x4 bv = decode_x16(bw[t][nf]);
                    const float sv =
                        __uint_as_float(t ? (sw[nf] & 0xFFFF0000u) : (sw[nf] << 16)) * 0.0625f;
#pragma unroll
                    for (int mf = 0; mf < MF; ++mf) {
                        const f32x4 p = mfma(xa[mf], bv, zero);
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            tot[mf][nf][r] = fmaf(sv, p[r], tot[mf][nf][r]);
                    }
                    // keep one N fragment's products live at a time
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            return;   // (a stage's code and scale reads are not hoisted into the one before)
        }
        u32x2 bw[NF];
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
            bw[nf] = *reinterpret_cast<const u32x2*>(slot + boff + nf * 16 * kBRow);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            u32x4 xa[MF];
#pragma unroll
            for (int mf = 0; mf < MF; ++mf)
                xa[mf] = *reinterpret_cast<const u32x4*>(slot + (t ? aoff1 : aoff0) +
                                                         mf * 16 * kARow);
#pragma unroll
            for (int nf = 0; nf < NF; ++nf) {
                const u32x4 bv = decode_x16(bw[nf][t]);
#pragma unroll
                for (int mf = 0; mf < MF; ++mf)
                    acc[mf][nf] = mfma(xa[mf], bv, (FIRST && t == 0) ? zero : acc[mf][nf]);
            }
        }
    };
    // Two stages (slots SL0, SL0 + 1), four 32-wide steps, each step's
    // activation fragments read one step ahead (MF = 8 only).
    auto compute_pair = [&](auto slc, bool first) {
        constexpr int SL0 = decltype(slc)::value;
        const uint8_t* sa = ring + SL0 * S::SLOT;
        const uint8_t* sb = ring + (SL0 + 1) * S::SLOT;
        auto read_a = [&](const uint8_t* slot, int off, u32x4 (&xa)[MF]) {
#pragma unroll
            for (int mf = 0; mf < MF; ++mf)
                xa[mf] = *reinterpret_cast<const u32x4*>(slot + off + mf * 16 * kARow);
        };
        auto read_b = [&](const uint8_t* slot, u32x2 (&bw)[NF]) {
#pragma unroll
            for (int nf = 0; nf < NF; ++nf)
                bw[nf] = *reinterpret_cast<const u32x2*>(slot + boff + nf * 16 * kBRow);
        };
        auto mstep = [&](const u32x4 (&xa)[MF], const u32x2 (&bw)[NF], int t, bool zero_acc) {
#pragma unroll
            for (int nf = 0; nf < NF; ++nf) {
                const u32x4 bv = decode_x16(bw[nf][t]);
#pragma unroll
                for (int mf = 0; mf < MF; ++mf)
                    acc[mf][nf] = mfma(xa[mf], bv, zero_acc ? zero : acc[mf][nf]);
            }
        };
        u32x4 xa0[MF], xa1[MF];
        u32x2 bw0[NF], bw1[NF];
        read_b(sa, bw0);
        read_a(sa, aoff0, xa0);
        read_a(sa, aoff1, xa1);
        if (first)
            mstep(xa0, bw0, 0, true);
        else
            mstep(xa0, bw0, 0, false);
        read_b(sb, bw1);
        read_a(sb, aoff0, xa0);
        mstep(xa1, bw0, 1, false);
        read_a(sb, aoff1, xa1);
        mstep(xa0, bw1, 0, false);
        mstep(xa1, bw1, 1, false);
    };
    // fold the finished group g into the totals
    auto close_group = [&](int g) {
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) {
            const float sv = bf16_to_f32(scrow[nf * 16 * a.G + g]) * 0.0625f;
#pragma unroll
            for (int mf = 0; mf < MF; ++mf)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    tot[mf][nf][r] = fmaf(sv, acc[mf][nf][r], tot[mf][nf][r]);
        }
    };
    // P stages s0 .. s0 + P - 1 (slots SL0 ..) per barrier; a group spans
    // whole P-stage steps (group >= 128 = 2 stages; P <= 2)
    auto step = [&](int s0, auto slc) {
        constexpr int SL0 = decltype(slc)::value * P;
        // stages issued after s0 + P - 1 by this wave
        wait_stage<S::LOADS, SLOTS - 2 * P>(stages - P - s0);
        // every wave's DMA of these stages has landed, and every wave has
        // finished the previous P stages, whose slots the next issue refills
        ring_barrier();
        const bool first = !G32 && (s0 * kStage) % a.group == 0;
        if (first && s0 > 0) close_group((s0 * kStage) / a.group - 1);
        static_for<P>([&](auto ic) {
            constexpr int I = decltype(ic)::value;
            if (s0 + SLOTS - P + I < stages)
                issue(s0 + SLOTS - P + I, (SL0 + SLOTS - P + I) % SLOTS);
        });
        if constexpr (MF == 8 && P == 2 && !G32) {
            compute_pair(std::integral_constant<int, SL0>{}, first);
        } else {
            if (first)
                compute(std::integral_constant<int, SL0>{}, std::true_type{}, s0);
            else
                compute(std::integral_constant<int, SL0>{}, std::false_type{}, s0);
            static_for<P - 1>([&](auto ic) {
                constexpr int I = 1 + decltype(ic)::value;
                compute(std::integral_constant<int, SL0 + I>{}, std::false_type{}, s0 + I);
            });
        }
    };

    // Scales of the workgroup's rows: rows n0 .. n0 + BN - 1 are one
    // contiguous run of dwords (n0 * G is even), copied by 4-byte DMA ahead of
    // stage 0, so stage 0's wait covers them.  Lanes past the run re-read its
    // last dword into unused LDS; entries past row N only feed outputs that
    // are never stored.
    {
        const int ndw = (min(S::BN, a.N - n0) * a.G + 1) / 2;
        const uint8_t* sb = reinterpret_cast<const uint8_t*>(a.scales + (size_t)n0 * a.G);
        const uint32_t sl = lds_addr(sc);
        for (int i = wave_id; i < (ndw + 63) / 64; i += 4 * KS)
            dma4((uint32_t)(4 * min(64 * i + lane, ndw - 1)), sb, sl + 256 * i);
    }
    const int pro = stages < SLOTS - P ? stages : SLOTS - P;
    for (int st = 0; st < pro; ++st) issue(st, st);

    // stage st lives in slot st % SLOTS: unrolled by SLOTS so that every slot
    // offset is a constant (stages is a multiple of 4, so of P)
    for (int st0 = 0; st0 < stages; st0 += SLOTS)
        static_for<SLOTS / P>([&](auto slc) {
            const int s0 = st0 + P * decltype(slc)::value;
            if (s0 < stages) step(s0, slc);
        });

    // the last group closes after one more barrier
    ring_barrier();
    if (!G32) close_group(G - 1);

    // K groups 1 .. KS - 1 leave their partial blocks in their own rings (all
    // their stages are consumed: every wave is past the barrier above), and
    // K group 0 adds them in group order
    if (KS > 1) {
        if (kg > 0) {
            f32x4* part = reinterpret_cast<f32x4*>(ring) + (wave * MF * NF) * 64 + lane;
#pragma unroll
            for (int mf = 0; mf < MF; ++mf)
#pragma unroll
                for (int nf = 0; nf < NF; ++nf) part[(mf * NF + nf) * 64] = tot[mf][nf];
        }
        __syncthreads();
        if (kg == 0) {
#pragma unroll
            for (int q = 1; q < KS; ++q) {
                const f32x4* part = reinterpret_cast<const f32x4*>(rings + q * (SLOTS * S::SLOT)) +
                                    (wave * MF * NF) * 64 + lane;
#pragma unroll
                for (int mf = 0; mf < MF; ++mf)
#pragma unroll
                    for (int nf = 0; nf < NF; ++nf) tot[mf][nf] += part[(mf * NF + nf) * 64];
            }
        }
    }

    // Output: every DMA was waited for in the last iteration, so once all
    // waves are past the barrier above the ring is free.  The fragments go to
    // LDS in the output dtype, then each thread writes whole 16-byte pieces of
    // output rows (fragment-order stores would fill a quarter of each line).
    const bool f32 = a.ydt == W4_F32;
    const int esz = f32 ? 4 : 2;
    uint8_t* ostage = rings;   // K group 0's ring
    constexpr int PMF = MF / S::OUT_PARTS;    // fragments of rows per staged part
    constexpr int PBM = S::BM / S::OUT_PARTS;
    static_for<S::OUT_PARTS>([&](auto hc) {
        constexpr int H = decltype(hc)::value;
        if (H > 0) __syncthreads();           // the previous part is stored
        if (kg == 0) {
#pragma unroll
            for (int mf = 0; mf < PMF; ++mf)
#pragma unroll
                for (int nf = 0; nf < NF; ++nf)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        uint8_t* p = ostage + (16 * mf + 4 * lk + r) * S::OUT_ROW +
                                     (wave * S::WN + 16 * nf + li) * esz;
                        const float v = tot[H * PMF + mf][nf][r];
                        if (f32)
                            *reinterpret_cast<float*>(p) = v;
                        else
                            *reinterpret_cast<uint16_t*>(p) = (uint16_t)f32_to_bf16_rne(v);
                    }
        }
        __syncthreads();
        const int per = 16 / esz;                 // elements per 16-byte piece
        const int cpr = S::BN / per;              // pieces per row
        for (int e = tid; e < PBM * cpr; e += S::THREADS) {
            const int row = e / cpr, c = e - row * cpr;
            const int m = m0 + H * PBM + row;
            if (m >= a.M) break;                  // rows only grow with e
            const int n = n0 + c * per;
            if (n >= a.N) continue;
            const u32x4 v = *reinterpret_cast<const u32x4*>(ostage + row * S::OUT_ROW + 16 * c);
            uint8_t* dst = static_cast<uint8_t*>(a.Y) + ((size_t)m * a.ldy + n) * esz;
            if (a.vec_out && n + per <= a.N) {
                gstore(reinterpret_cast<u32x4*>(dst), v);
            } else {
                for (int i = 0; i < per && n + i < a.N; ++i) {
                    if (f32)
                        gstore(reinterpret_cast<uint32_t*>(dst) + i, v[i]);
                    else
                        gstore(reinterpret_cast<uint16_t*>(dst) + i,
                               (uint16_t)(v[i >> 1] >> (16 * (i & 1))));
                }
            }
        }
    });
}

// Shared decode (groups of 64 or more): WM x WN waves, each computing
// 64 x 48 outputs (MF = 4, NF = 3) of a (64 WM) x (48 WN) block.  Above, each
// wave decodes the code words of its own 48 weight rows, so the WM waves of
// a block that share those rows would decode every word WM times; here the
// workgroup decodes each word of a stage once, into an LDS buffer of bf16
// values laid out like an activation tile, and every wave reads its B
// fragments from there.  Per 64-wide K stage:
//   - each wave's DMA fills its share of the stage's activation tile (16-byte
//     loads) and of its code tile (4-byte loads, U per wave); lane i of a
//     code load brings exactly the word that lane i decodes, so a lane needs
//     only its own wave's loads to have landed before decoding;
//   - stage s + 1 is decoded (into one of two buffers) while stage s is
//     multiplied from the other: one barrier per stage publishes the decoded
//     words and the stage's activation tile, and frees the slot and buffer
//     that the next DMA and decode overwrite;
//   - the products, their K permutation (step t of lane group j takes words
//     2j + t) and the per-group scaling are those of prefill_kernel, so the
//     two give the same bits.
// Decoded row i: 128 bytes, position p holds word p ^ g(i) (the activation
// swizzle), so both the 16-byte decode writes (16 rows, one word each per
// lane group) and the fragment reads are free of bank conflicts.
template <int WM, int WN, int SLOTS>
struct SdShape {
    static constexpr int NW = WM * WN;
    static constexpr int THREADS = 64 * NW;
    static constexpr int BM = 64 * WM;
    static constexpr int BN = 48 * WN;
    static constexpr int A_BYTES = BM * kARow;
    static constexpr int B_BYTES = BN * kBRow;
    static constexpr int SLOT = A_BYTES + B_BYTES;
    static constexpr int DEC = BN * kARow;               // one decoded stage
    static constexpr int A_DMA = A_BYTES / 1024 / NW;    // 16-byte DMA per wave per stage
    static constexpr int U = B_BYTES / 256 / NW;         // 4-byte DMA per wave per stage
    static constexpr int LOADS = A_DMA + U;
    static_assert(A_DMA * NW * 1024 == A_BYTES, "activation tile: whole DMA rounds per wave");
    static_assert(U * NW * 256 == B_BYTES, "code tile: whole DMA rounds per wave");
    static_assert(SLOTS >= 3 && SLOTS % 2 == 0, "a stage decoded ahead; buffer parity constant");
    static_assert(LOADS * (SLOTS - 1) < 64, "vmcnt range");
    static constexpr int LDS = SLOTS * SLOT + 2 * DEC;
    static constexpr int OUT_ROW = BN * 4 + 16;          // padded fp32 staging row (bytes)
    static_assert(BM * OUT_ROW <= LDS, "output block staged whole");
};

// s_waitcnt lgkmcnt(0), vmcnt and expcnt left alone: this wave's LDS writes
// are done (the raw barrier does not wait for them)
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

template <int WM, int WN, int SLOTS>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(2)))
void shared_decode_kernel(PfArgs a) {
    using S = SdShape<WM, WN, SLOTS>;
    constexpr int MF = 4, NF = 3;
    __shared__ __align__(16) uint8_t lds[S::LDS];
    __shared__ __align__(16) uint16_t sc[S::BN * kMaxG];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, wn = wave / WM;
    const int li = lane & 15, lk = lane >> 4;

    // XCD x = blockIdx % 8 runs every M block of N blocks x, x + 8, ...
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int mb = j % a.m_blocks;
    const int nb = (j / a.m_blocks) * 8 + xcd;
    if (nb >= a.n_blocks) return;
    const int m0 = mb * S::BM, n0 = nb * S::BN;
    const int KW = a.K / 8;
    const int stages = a.K / kStage;

    uint32_t aoffs[S::A_DMA];
#pragma unroll
    for (int d = 0; d < S::A_DMA; ++d) {
        const int r = 8 * (wave * S::A_DMA + d) + (lane >> 3);
        const int q = (lane & 7) ^ swz_a(r);
        const int m = min(m0 + r, a.M - 1);
        aoffs[d] = (uint32_t)(((size_t)m * a.ldx + 8 * q) * 2);
    }
    // decode unit q (U per wave): rows 16 (q / 2) .. + 15, words 4 (q % 2) + lk
    uint32_t boffs[S::U];
    int doff[S::U];
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
        const int q = wave * S::U + u;
        const int row = 16 * (q >> 1) + li;
        const int word = 4 * (q & 1) + lk;
        const int n = min(n0 + row, a.N - 1);
        boffs[u] = (uint32_t)(((size_t)n * KW + word) * 4);
        doff[u] = row * kARow + 16 * (word ^ swz_a(row));
    }
    const uint32_t lds0 = lds_addr(lds);
    const uint32_t adst = lds0 + 1024 * (wave * S::A_DMA);
    const uint32_t bdst = lds0 + S::A_BYTES + 256 * (wave * S::U);
    const int bsrc = S::A_BYTES + 256 * (wave * S::U) + 4 * lane;   // this lane's code word
    auto issue = [&](int st, int slot) {
        const uint8_t* ab = reinterpret_cast<const uint8_t*>(a.X) + (size_t)st * kStage * 2;
        const uint8_t* bb = reinterpret_cast<const uint8_t*>(a.codes) + (size_t)st * kStage / 2;
#pragma unroll
        for (int d = 0; d < S::A_DMA; ++d) dma16(aoffs[d], ab, adst + slot * S::SLOT + 1024 * d);
#pragma unroll
        for (int u = 0; u < S::U; ++u) dma4(boffs[u], bb, bdst + slot * S::SLOT + 256 * u);
    };
    uint8_t* const dec = lds + SLOTS * S::SLOT;
    auto decode = [&](auto slc, auto bufc) {
        constexpr int SL = decltype(slc)::value, BUF = decltype(bufc)::value;
        uint32_t w[S::U];
#pragma unroll
        for (int u = 0; u < S::U; ++u)
            w[u] = *reinterpret_cast<const uint32_t*>(lds + SL * S::SLOT + bsrc + 256 * u);
#pragma unroll
        for (int u = 0; u < S::U; ++u)
            *reinterpret_cast<u32x4*>(dec + BUF * S::DEC + doff[u]) = decode_x16(w[u]);
    };

    // fragment offsets: step t of lane group lk reads word 2 lk + t of row li
    const int gl = swz_a(li);
    const int foff0 = li * kARow + 16 * ((2 * lk) ^ gl);
    const int foff1 = li * kARow + 16 * ((2 * lk + 1) ^ gl);
    const int arow = 64 * wm * kARow, brow = 48 * wn * kARow;
    const uint16_t* scrow = sc + (48 * wn + li) * a.G;

    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 tot[MF][NF], acc[MF][NF];
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) tot[mf][nf] = zero;

    // one 32-wide step's fragments: MF activation, NF decoded weight
    struct Frags {
        u32x4 a[MF], b[NF];
    };
    auto read_frags = [&](auto slc, auto bufc, int fo, Frags& f) {
        constexpr int SL = decltype(slc)::value, BUF = decltype(bufc)::value;
        const uint8_t* sa = lds + SL * S::SLOT + arow;
        const uint8_t* sb = dec + BUF * S::DEC + brow;
#pragma unroll
        for (int mf = 0; mf < MF; ++mf)
            f.a[mf] = *reinterpret_cast<const u32x4*>(sa + fo + mf * 16 * kARow);
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
            f.b[nf] = *reinterpret_cast<const u32x4*>(sb + fo + nf * 16 * kARow);
    };
    // a group's first step starts its MFMA chains from a zero operand
    auto mstep = [&](const Frags& f, auto zc) {
        constexpr bool Z = decltype(zc)::value;
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
#pragma unroll
            for (int mf = 0; mf < MF; ++mf)
                acc[mf][nf] = mfma(f.a[mf], f.b[nf], Z ? zero : acc[mf][nf]);
    };
    auto close_group = [&](int g) {
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) {
            const float sv = bf16_to_f32(scrow[nf * 16 * a.G + g]) * 0.0625f;
#pragma unroll
            for (int mf = 0; mf < MF; ++mf)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    tot[mf][nf][r] = fmaf(sv, acc[mf][nf][r], tot[mf][nf][r]);
        }
    };

    // scales of the block's rows, ahead of stage 0 (as in prefill_kernel)
    {
        const int ndw = (min(S::BN, a.N - n0) * a.G + 1) / 2;
        const uint8_t* sb = reinterpret_cast<const uint8_t*>(a.scales + (size_t)n0 * a.G);
        const uint32_t sl = lds_addr(sc);
        for (int i = wave; i < (ndw + 63) / 64; i += S::NW)
            dma4((uint32_t)(4 * min(64 * i + lane, ndw - 1)), sb, sl + 256 * i);
    }
    const int pro = stages < SLOTS ? stages : SLOTS;
    for (int st = 0; st < pro; ++st) issue(st, st);
    // this wave's loads of stage 0 (and of the scales) have landed
    wait_stage<S::LOADS, SLOTS - 1>(stages - 1);
    asm volatile("" ::: "memory");
    decode(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
    wait_lgkm0();
    ring_barrier();
    Frags f0, f1;
    read_frags(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, foff0, f0);

    // Stage s lives in slot s % SLOTS and is decoded into buffer s % 2
    // (unrolled by SLOTS so that both are constants).  Software pipeline, per
    // stage: read step 1's fragments; multiply step 0; decode stage s + 1
    // (this wave's loads of it have landed); one barrier publishes every
    // wave's decode and activation tile of stage s + 1 and proves stage s
    // read by all, so its slot is refilled with stage s + SLOTS; read stage
    // s + 1's step 0 fragments; multiply step 1.  The step-0 products are
    // still in the matrix cores across the decode and the barrier.
    const int spg = a.group / kStage;   // stages per scale group
    int gs = 0, gi = 0;                 // stage within its group, group index
    for (int st0 = 0; st0 < stages; st0 += SLOTS)
        static_for<SLOTS>([&](auto ic) {
            constexpr int I = decltype(ic)::value;
            constexpr int NX = (I + 1) % SLOTS, BX = (I + 1) % 2;
            const int s = st0 + I;
            if (s >= stages) return;
            read_frags(ic, std::integral_constant<int, I % 2>{}, foff1, f1);
            if (gs == 0)
                mstep(f0, std::true_type{});
            else
                mstep(f0, std::false_type{});
            if (s + 1 < stages) {
                // stages issued after s + 1 may still be in flight
                wait_stage<S::LOADS, SLOTS - 2>(stages - s - 2);
                asm volatile("" ::: "memory");
                decode(std::integral_constant<int, NX>{}, std::integral_constant<int, BX>{});
            }
            wait_lgkm0();
            ring_barrier();
            if (s + SLOTS < stages) issue(s + SLOTS, I);
            if (s + 1 < stages)
                read_frags(std::integral_constant<int, NX>{}, std::integral_constant<int, BX>{},
                           foff0, f0);
            mstep(f1, std::false_type{});
            if (++gs == spg) {
                close_group(gi++);
                gs = 0;
            }
        });

    // Output through LDS as whole 16-byte row pieces (every DMA was waited
    // for; past the barrier no wave reads the ring)
    const bool f32 = a.ydt == W4_F32;
    const int esz = f32 ? 4 : 2;
    __syncthreads();
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint8_t* p = lds + (64 * wm + 16 * mf + 4 * lk + r) * S::OUT_ROW +
                             (48 * wn + 16 * nf + li) * esz;
                const float v = tot[mf][nf][r];
                if (f32)
                    *reinterpret_cast<float*>(p) = v;
                else
                    *reinterpret_cast<uint16_t*>(p) = (uint16_t)f32_to_bf16_rne(v);
            }
    __syncthreads();
    const int per = 16 / esz;
    const int cpr = S::BN / per;
    for (int e = tid; e < S::BM * cpr; e += S::THREADS) {
        const int row = e / cpr, c = e - row * cpr;
        const int m = m0 + row;
        if (m >= a.M) break;
        const int n = n0 + c * per;
        if (n >= a.N) continue;
        const u32x4 v = *reinterpret_cast<const u32x4*>(lds + row * S::OUT_ROW + 16 * c);
        uint8_t* dst = static_cast<uint8_t*>(a.Y) + ((size_t)m * a.ldy + n) * esz;
        if (a.vec_out && n + per <= a.N) {
            gstore(reinterpret_cast<u32x4*>(dst), v);
        } else {
            for (int i = 0; i < per && n + i < a.N; ++i) {
                if (f32)
                    gstore(reinterpret_cast<uint32_t*>(dst) + i, v[i]);
                else
                    gstore(reinterpret_cast<uint16_t*>(dst) + i,
                           (uint16_t)(v[i >> 1] >> (16 * (i & 1))));
            }
        }
    }
}

struct PfCfg {
    int MF, NF, slots, per_barrier, ks;
};
// 64 x 192, 64 x 128 or 64 x 64 blocks; ring slots; stages per barrier; K
// groups.  Measured at N = 12288, K = 1536, g256: two stages per barrier beat
// one (the per-barrier latency chain, not the DMA depth, bounds the loop).
// Entries 0, 10, 6 and 1 are the unsplit block shapes chosen below (10: the
// 64 x 128 block with a three-slot ring, three workgroups per CU); entries 2
// and 3 are the one-stage variants, kept for comparison runs; entries 4 and
// 5 split K over three or two wave groups.  Entry 9 is the shared-decode
// kernel (128 x 192 blocks of eight waves; its MF and NF give the block as
// for the others: 16 MF rows, 64 NF columns).
constexpr PfCfg kPfCfgs[] = {{4, 3, 4, 2, 1}, {4, 1, 6, 2, 1}, {4, 3, 5, 1, 1},
                             {4, 1, 5, 1, 1}, {4, 1, 4, 2, 3}, {4, 1, 6, 2, 2},
                             {4, 2, 4, 2, 1}, {8, 3, 6, 2, 1}, {8, 2, 3, 1, 1},
                             {8, 3, 4, 1, 1}, {4, 2, 3, 1, 1}};
constexpr int kPfShared = 9;
constexpr int kPfNumCfgs = sizeof(kPfCfgs) / sizeof(kPfCfgs[0]);

struct PfPlan {
    int cfg, BM, BN, m_blocks, n_blocks, grid;
};

// Unsplit block shape.  Each candidate holds a fixed number of workgroups
// per CU (LDS and registers), so a launch runs in rounds of that many times
// the CUs; choose the fewest rounds times the measured time of one full
// round, wider blocks on ties.  Groups of 64 or more, N = 12288, K = 1536,
// g256: 64 x 192 blocks two per CU 27.6 us; 64 x 128 three per CU (a
// three-slot ring, three waves per SIMD) 26.5 us, the same outputs per round
// as 64 x 192 (M = 512: 29.1 against 30.3 us, M = 1024: 53.1 against 56.0,
// measured side by side); 64 x 128 two per CU 20.9 us; 64 x 64 two per CU
// 14.1 us.  At N = 12288 this gives 64 x 64 for 65..128 rows, 64 x 128 two
// per CU for 129..320 and 513..640, three per CU for 321..512 and from 641.
// Group 32 (a scale per MFMA step: more registers and ALU work per block)
// has no 64 x 192 entry, which spills, and its own round times (64 x 128
// three per CU 35.5 us, two per CU 26 us, 64 x 64 17.5 us): 64 x 64 up to
// 128 rows, 64 x 128 two per CU for 129..320, three per CU above (512 rows
// 35.5 against 39.7 us two per CU, 1024 rows 65.1 against 70.5).
struct PfCand {
    int cfg, BN, per_cu;
    double t_round;
};
static int pick_block_cfg(int M, int N, int group) {
    static const PfCand kCand[4] = {
        {0, 192, 2, 27.6}, {10, 128, 3, 26.5}, {6, 128, 2, 20.9}, {1, 64, 2, 14.1}};
    static const PfCand kCand32[3] = {{10, 128, 3, 35.5}, {6, 128, 2, 26.0}, {1, 64, 2, 17.5}};
    const PfCand* cand = group == 32 ? kCand32 : kCand;
    const int ncand = group == 32 ? 3 : 4;
    const long long mb = (M + 63) / 64;
    int best = 0;
    double best_t = 1e300;
    for (int i = 0; i < ncand; ++i) {
        const PfCand& c = cand[i];
        const long long slots = (long long)c.per_cu * kNumCUs;
        const long long wgs = mb * ((N + c.BN - 1) / c.BN);
        const double t = (double)((wgs + slots - 1) / slots) * c.t_round;
        if (t < best_t - 1e-9) {   // candidates in decreasing width: ties keep the wider
            best_t = t;
            best = c.cfg;
        }
    }
    return best;
}

PfPlan plan_prefill(int M, int N, int K, int group) {
    PfPlan p;
    p.cfg = pick_block_cfg(M, N, group);
    // 64 x 64 blocks that leave CUs idle (at most one workgroup per CU)
    // split K over three or two wave groups.  Measured
    // at N = 12288, K = 1536, g256: 64 rows 11.8 -> 9.0 us, 32 rows 11.6 ->
    // 8.7 us; at 128 rows (768 workgroup slots wanted, one per CU fits) the
    // split is slower (14.4 -> 16.6 us).
    const int G = K / group;
    // Group 32 splits two ways at K = 1536: its three-way split spills
    // registers (M = 64: 11.7 us against 12.3 us, unsplit 15.7 us); at
    // K = 6144 (96 stages) three ways still wins for few rows (M = 64: 32.5
    // against 35.7 us; equal at 256 and 512).
    if (p.cfg == 1 && (M + 63) / 64 * ((N + 63) / 64) <= kNumCUs)
        p.cfg = G % 3 == 0 && (group != 32 || G > kMaxG32) ? 4 : (G % 2 == 0 ? 5 : 1);
    const int o = config()->prefill_cfg;  // W4_PREFILL_CFG: a kPfCfgs index
    if (o >= 0 && o < kPfNumCfgs) p.cfg = o;
    // a K split needs whole scale groups per wave group
    if (G % kPfCfgs[p.cfg].ks != 0) p.cfg = 1;   // the split entries are 64 x 64 blocks
    // group 32 beyond 48 groups: only the split workgroups hold the scale table
    // (G is a multiple of 8 here, so the two-way split divides it)
    if (group == 32 && G > kMaxG32 && kPfCfgs[p.cfg].ks == 1) p.cfg = 5;
    // the wide tiles and the shared decode are for groups of 64 or more
    if (group == 32 && (p.cfg == 7 || p.cfg == 8 || p.cfg == kPfShared)) p.cfg = 6;
    p.BM = 16 * kPfCfgs[p.cfg].MF;
    p.BN = 64 * kPfCfgs[p.cfg].NF;
    p.m_blocks = (M + p.BM - 1) / p.BM;
    p.n_blocks = (N + p.BN - 1) / p.BN;
    p.grid = 8 * p.m_blocks * ((p.n_blocks + 7) / 8);
    return p;
}

}  // namespace

bool prefill_supported(int M, int N, int K, int group, int ldx) {
    // per-lane DMA offsets are 32-bit: activation rows and code rows must be
    // addressable from their buffer's start within 4 GiB
    const size_t x_span = ((size_t)(M - 1) * (size_t)ldx + (size_t)K) * 2;
    const size_t c_span = (size_t)N * (size_t)K / 2;
    // group 32: K a multiple of 256 as for group 256, so that every K group
    // of every split holds an even number of stages (whole two-stage steps)
    const bool groups_fit = group == 32 ? K % 256 == 0 && K / group <= kMaxG32Split
                                        : group % kStage == 0 && K / group <= kMaxG;
    return groups_fit && K % kStage == 0 &&
           x_span < (1ull << 32) && c_span < (1ull << 32);
}

template <bool G32>
static void launch_cfg(int cfg, dim3 g, dim3 b, hipStream_t s, const PfArgs& a) {
    switch (cfg) {
        case 0: prefill_kernel<4, 3, 4, 2, 1, G32><<<g, b, 0, s>>>(a); break;
        case 1: prefill_kernel<4, 1, 6, 2, 1, G32><<<g, b, 0, s>>>(a); break;
        case 2: prefill_kernel<4, 3, 5, 1, 1, G32><<<g, b, 0, s>>>(a); break;
        case 3: prefill_kernel<4, 1, 5, 1, 1, G32><<<g, b, 0, s>>>(a); break;
        case 4: prefill_kernel<4, 1, 4, 2, 3, G32><<<g, b, 0, s>>>(a); break;
        case 5: prefill_kernel<4, 1, 6, 2, 2, G32><<<g, b, 0, s>>>(a); break;
        case 7:
            if constexpr (!G32) {
                prefill_kernel<8, 3, 6, 2, 1, false><<<g, b, 0, s>>>(a);
                break;
            }
            [[fallthrough]];
        case 8:
            if constexpr (!G32) {
                prefill_kernel<8, 2, 3, 1, 1, false><<<g, b, 0, s>>>(a);
                break;
            }
            [[fallthrough]];
        case 10: prefill_kernel<4, 2, 3, 1, 1, G32><<<g, b, 0, s>>>(a); break;
        case kPfShared:
            if constexpr (!G32) {
                shared_decode_kernel<2, 4, 4><<<g, dim3(SdShape<2, 4, 4>::THREADS), 0, s>>>(a);
                break;
            }
            [[fallthrough]];
        default: prefill_kernel<4, 2, 4, 2, 1, G32><<<g, b, 0, s>>>(a); break;
    }
}

int launch_prefill(const void* packed, int N, int K, int group, int M, const uint16_t* X,
                   int ldx, void* Y, int ldy, int ydt, hipStream_t s) {
    const PfPlan p = plan_prefill(M, N, K, group);
    PfArgs a;
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
    const size_t esz = ydt == W4_F32 ? 4 : 2;
    a.vec_out = (reinterpret_cast<uintptr_t>(Y) % 16 == 0) && ((size_t)ldy * esz) % 16 == 0;
    const dim3 g(p.grid), b(256 * kPfCfgs[p.cfg].ks);
    if (group == 32)
        launch_cfg<true>(p.cfg, g, b, s, a);
    else
        launch_cfg<false>(p.cfg, g, b, s, a);
    return hip_fail(hipGetLastError(), "prefill launch");
}

void describe_prefill(int M, int N, int K, int group, char* buf, size_t len) {
    const PfPlan p = plan_prefill(M, N, K, group);
    if (p.cfg == kPfShared) {
        snprintf(buf, len,
                 "mfma 16x16x32 dma-ring shared-decode block %dx%d waves 2x4 slots %d stage %d "
                 "grid=%d (K=%d g=%d)",
                 p.BM, p.BN, kPfCfgs[p.cfg].slots, kStage, p.grid, K, group);
        return;
    }
    snprintf(buf, len,
             "mfma 16x16x32 dma-ring block %dx%d waves %dx4 slots %d stage %d x%d grid=%d (K=%d g=%d)",
             p.BM, p.BN, kPfCfgs[p.cfg].ks, kPfCfgs[p.cfg].slots, kStage,
             kPfCfgs[p.cfg].per_barrier, p.grid, K, group);
}

}  // namespace w4
