// w4_ordered.hip -- the decode-ordered persistent kernel (W4_SWEEP_PERSISTENT).
//
// [P1] "Gemma 4 E2B on a 4 GB GPU with plain PyTorch, faster than llama.cpp",
// paragraph on the decode step captured once as a graph and replayed per
// token: a step is a fixed chain of GEMVs, each reading what the previous one
// wrote.  Ordering rule: no output of op i+1 is computed, and no activation of
// op i+1 is read, before every output of op i is written.
//
// One workgroup per CU, 8 waves.  Each op's rows are split into one
// contiguous share per workgroup.  On MI355X a grid-wide handoff (outputs
// visible, every workgroup told) costs ~3 us against 0.2-1.3 us of HBM time
// per layer op, so everything that does not depend on the previous op is
// taken off that path:
//  - weights never depend on activations: wave 7, the DMA wave, copies the
//    workgroup's share of a later resident op (codes and scales, up to 56 KB)
//    into one of two LDS slots, so an op's compute reads its weights from
//    LDS.  It issues the copy when the op before that one starts computing:
//    the copy's HBM traffic then overlaps compute that reads only LDS, not the
//    handoff's stores, polls and loads (issued at the end of the previous op
//    it slowed each handoff by ~0.6 us), and the issue, which stalls while
//    every CU copies at once, delays no compute wave;
//  - waves 0..6 compute a resident share: each row's chunks are cut into
//    parts that 16-lane groups take (the host's plan), so that shares of a
//    few rows still keep every compute wave busy;
//  - wave 0 is the control wave: it issues no DMA (so its waits cover only
//    its own accesses), polls the completion counters, loads the activation
//    (agent scope, 16-byte loads) into LDS for the whole workgroup, adds the
//    partial sums, stores the workgroup's outputs (agent scope), waits for
//    them to complete and signals;
//  - the activation is multiplied as it is, bf16, against the exact bf16
//    decode of the codes (w4_common.h): no conversion pass and no range
//    fallback, so one barrier per op separates the handoff from the compute;
//  - completion is counted in eight counters, one per XCD's workgroups
//    (workgroup b runs on XCD b mod 8), each in its own 128-byte line: eight
//    adders per address instead of one counter for all (measured 1.9 us
//    against 3.7 us per bare handoff; per-workgroup flags polled as a whole
//    3.6 us).
// Shares too large for a slot (the 262144-row output layer: 885 KB per
// workgroup) are streamed from HBM by all 8 waves after the handoff, with the
// next row group in flight.
//
// Safety: every wait is bounded; a wait that gives up sets the error word
// and returns, and every other wait then gives up too, so the grid drains.
// The last workgroup to finish a replay resets the counters for the next one
// (every workgroup has made its last read of them by then).  Launches of one
// handle must not overlap.
#include "w4_gemv_core.h"
#include "w4_persist.h"
#include "w4_ring.h"

namespace w4 {

namespace {

using namespace ring;

constexpr unsigned kOrdSpin = 1u << 20;

// Dynamic LDS layout of a workgroup.
constexpr int kSlotBytes = kOrdCodeBytes + kOrdScaleBytes;
// The activation copy is quarter-major: 16-byte quarter q of chunk c (32
// elements, 64 bytes) sits at q * kQStride + 16 c, so lanes that touch
// consecutive chunks touch consecutive 16-byte words (a chunk-major copy puts
// them 64 bytes apart, on the same LDS banks).
constexpr int kQStride = (kOrdMaxK / 32) * 16;
constexpr int kXbOff = 2 * kSlotBytes;                  // bf16 activation pairs
constexpr int kOutOff = kXbOff + kOrdMaxK * 2;          // the share's partial sums (fp32)
constexpr int kFlagOff = kOutOff + kOrdMaxPartials * 4; // flags and the LDS count
constexpr int kOrdLds = kFlagOff + 16;

// Rows [w N / G, (w + 1) N / G) of workgroup w (floor division), in 32-bit
// arithmetic: w N / G = w (N / G) + w (N % G) / G, and w (N % G) < G^2.
__device__ __forceinline__ int share_start(int N, int w, int G) {
    const unsigned q = (unsigned)N / (unsigned)G, r = (unsigned)N % (unsigned)G;
    return (int)((unsigned)w * q + ((unsigned)w * r) / (unsigned)G);
}
__device__ __forceinline__ void share_rows(int N, int w, int G, int& rb, int& re) {
    rb = share_start(N, w, G);
    re = share_start(N, w + 1, G);
}

// wait until at most n of this wave's DMA loads are in flight (0 <= n < 64;
// larger n waits for all)
__device__ __forceinline__ void wait_vm_rt(int n) {
    switch (n) {
#define W4_CASE(N) case N: wait_vm<N>(); break;
#define W4_CASE8(B) W4_CASE(B) W4_CASE(B + 1) W4_CASE(B + 2) W4_CASE(B + 3) \
                    W4_CASE(B + 4) W4_CASE(B + 5) W4_CASE(B + 6) W4_CASE(B + 7)
        W4_CASE8(0) W4_CASE8(8) W4_CASE8(16) W4_CASE8(24)
        W4_CASE8(32) W4_CASE8(40) W4_CASE8(48) W4_CASE8(56)
#undef W4_CASE8
#undef W4_CASE
        default: wait_vm<0>(); break;
    }
}

// Issue the DMA of op's share for workgroup w into `slot`, 1 KB per
// instruction (16 bytes per lane).  Codes [rb K/2, re K/2) and scales
// [rb G 2, re G 2) are contiguous byte ranges, whole 16-byte units for a
// resident op (K % 256 == 0 and G % 8 == 0, checked on the host); lanes past
// a range re-read its last 16 bytes into slot space past the share (the
// slot's code and scale areas are whole kilobytes).  An empty share issues
// nothing.
__device__ __forceinline__ void issue_share(const SweepOp& op, int w, int G, uint8_t* slot,
                                            int lane) {
    int rb, re;
    share_rows(op.N, w, G, rb, re);
    const int K = op.C * 32;
    const uint32_t cb = (uint32_t)(re - rb) * (uint32_t)(K / 2);
    const uint32_t c0 = (uint32_t)rb * (uint32_t)(K / 2);
    const int nc = (int)((cb + 1023u) / 1024u);
    const uint32_t lds0 = lds_addr(slot);
    for (int d = 0; d < nc; ++d) {
        const uint32_t o = (uint32_t)d * 1024u + 16u * lane;
        const uint32_t src = c0 + (o < cb ? o : (cb >= 16u ? cb - 16u : 0u));
        dma16(src, op.codes, lds0 + (uint32_t)d * 1024u);
    }
    const uint32_t sb = (uint32_t)(re - rb) * (uint32_t)(op.G * 2);
    const uint32_t s0 = (uint32_t)rb * (uint32_t)(op.G * 2);
    const int ns = (int)((sb + 1023u) / 1024u);
    for (int d = 0; d < ns; ++d) {
        const uint32_t o = (uint32_t)d * 1024u + 16u * lane;
        const uint32_t src = s0 + (o < sb ? o : (sb >= 16u ? sb - 16u : 0u));
        dma16(src, op.scales, lds0 + kOrdCodeBytes + (uint32_t)d * 1024u);
    }
}

// DMA instructions issue_share issues for op's share of workgroup w
__device__ __forceinline__ int share_dmas(const SweepOp& op, int w, int G) {
    int rb, re;
    share_rows(op.N, w, G, rb, re);
    return ((re - rb) * (op.C * 16) + 1023) / 1024 + ((re - rb) * (op.G * 2) + 1023) / 1024;
}

// The activation (K = 32 C bf16, written by any CU) into the workgroup's
// quarter-major copy, by global-to-LDS DMA from one wave, then waited for:
// instruction j moves quarter j % 4 of chunks 64 (j / 4) + lane (16 bytes per
// lane, landing at consecutive LDS addresses).  The loads are agent scope
// (sc1: coherent across XCDs, as the compiler's own agent-scope loads are).
// Lanes past the last chunk re-read it into the unused tail of their quarter
// (256 chunks each), which nothing reads.  The caller has no other
// vector-memory access in flight that it needs to overlap.
__device__ __forceinline__ void dma16_agent(uint32_t off, const void* base, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 sc1"
                 :
                 : "v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void load_x_dma(const void* x, int C, int lane, uint8_t* smem) {
    const int nj = 4 * ((C + 63) / 64);
    for (int j = 0; j < nj; ++j) {
        int c = 64 * (j >> 2) + lane;
        c = c < C ? c : C - 1;
        dma16_agent(64u * (uint32_t)c + 16u * (uint32_t)(j & 3), x,
                    lds_addr(smem + kXbOff + (j & 3) * kQStride + 16 * 64 * (j >> 2)));
    }
}

// One lane's activation slice for tile (L, U) of a streamed share: chunks
// lk + L u of the workgroup's bf16 copy in LDS; chunks past the row end read
// as zero.  UT > 0: U is the compile-time UT; UT == 0: U at run time.
template <int L, int UT = 0>
__device__ __forceinline__ void slice_from_lds(const uint8_t* smem, int C, int U, int lk,
                                               uint32_t (&xr)[kPwMaxU][16]) {
#pragma unroll
    for (int u = 0; u < (UT > 0 ? UT : kPwMaxU); ++u) {
        const int c = lk + L * u;
        if ((UT > 0 || u < U) && c < C) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x4 v =
                    *reinterpret_cast<const u32x4*>(smem + kXbOff + i * kQStride + 16 * c);
                xr[u][4 * i + 0] = v[0];
                xr[u][4 * i + 1] = v[1];
                xr[u][4 * i + 2] = v[2];
                xr[u][4 * i + 3] = v[3];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) xr[u][i] = 0u;
        }
    }
}

// Row sum of one lane's chunks: q the codes, sc the scales (bf16 bits).
// Codes enter as the exact bf16 values 16 (c - 8) (w4_common.h), so the
// activations need no conversion; each chunk's sum is scaled by s / 16.
template <int UT = 0>
__device__ __forceinline__ float row_partial(const u32x4 (&q)[kPwMaxU], const uint32_t (&sc)[kPwMaxU],
                                             const uint32_t (&xr)[kPwMaxU][16], int U) {
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < (UT > 0 ? UT : kPwMaxU); ++u) {
        if (UT > 0 || u < U)
            acc = fmaf(bf16_to_f32(sc[u]) * 0.0625f, chunk_dot_x16(q[u], xr[u]), acc);
    }
    return acc;
}

// Resident share (rows 0 .. R-1 of the slot): tasks (part p, row r), a
// row's sum over part p's CP chunks, numbered t = p Rm + r (Rm the largest
// share's rows; rows r >= R are skipped).  The host's plan gives each 16-lane
// group of waves 0..6 a contiguous run of tasks (entry = first << 16 |
// count), balanced over the SIMDs.  Lane k of a group holds the activation of
// chunks c0 + k + 16 u of the current part (reloaded when the part changes);
// the next task's codes are read from the slot while the current one is
// multiplied.  A task's sum goes to the LDS buffer, entry r P + p.
template <int UP>
__device__ __forceinline__ void compute_resident(const SweepOp& op, const uint8_t* smem,
                                                 const uint8_t* slot, int R, int lane,
                                                 uint32_t entry) {
    const int n = (int)(entry & 0xFFFFu);
    if (n == 0 || R <= 0) return;
    const int lk = lane & 15;
    const int P = op.P, CP = op.CP, Rm = op.Rm;
    const int C = op.C, G = op.G, gshift = op.gshift, rowb = 16 * C;
    const int t0 = (int)(entry >> 16);
    float* part = reinterpret_cast<float*>(const_cast<uint8_t*>(smem) + kOutOff);
    const uint16_t* sslot = reinterpret_cast<const uint16_t*>(slot + kOrdCodeBytes);

    // chunk of lane lk for step u of part p; chunks past the part's end read
    // the part's first chunk (a valid address) against a zero activation
    auto chunk = [&](int p, int u) {
        const int c0 = p * CP;
        const int c = c0 + lk + 16 * u;
        return c < c0 + CP && c < C ? c : c0;
    };
    uint32_t xr[UP][16];
    auto load_x = [&](int p) {
#pragma unroll
        for (int u = 0; u < UP; ++u) {
            const int c0 = p * CP;
            const int c = c0 + lk + 16 * u;
            const bool in = c < c0 + CP && c < C;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (in) v = *reinterpret_cast<const u32x4*>(smem + kXbOff + i * kQStride + 16 * c);
                xr[u][4 * i + 0] = v[0];
                xr[u][4 * i + 1] = v[1];
                xr[u][4 * i + 2] = v[2];
                xr[u][4 * i + 3] = v[3];
            }
        }
    };
    auto load = [&](int p, int r, u32x4 (&qq)[UP], uint32_t (&ss)[UP]) {
        r = r < R ? r : R - 1;
#pragma unroll
        for (int u = 0; u < UP; ++u) {
            const int c = chunk(p, u);
            qq[u] = *reinterpret_cast<const u32x4*>(slot + (size_t)r * rowb + 16 * c);
            ss[u] = sslot[r * G + (c >> gshift)];
        }
    };
    auto finish = [&](int p, int r, const u32x4 (&qq)[UP], const uint32_t (&ss)[UP]) {
        float acc = 0.f;
#pragma unroll
        for (int u = 0; u < UP; ++u)
            acc = fmaf(bf16_to_f32(ss[u]) * 0.0625f, chunk_dot_x16(qq[u], xr[u]), acc);
        acc = group_sum<16>(acc);
        if (lk == 0 && r < R) part[r * P + p] = acc;
    };

    int p = t0 / Rm, r = t0 - p * Rm;
    int xp = p;
    load_x(p);
    u32x4 qa[UP], qb[UP];
    uint32_t sa[UP], sb[UP];
    load(p, r, qa, sa);
    int k = 0;
    while (true) {
        // the next task (or this one again on the last step)
        int pn = p, rn = r + 1;
        if (rn == Rm) {
            rn = 0;
            ++pn;
        }
        const bool more = k + 1 < n;
        load(more ? pn : p, more ? rn : r, qb, sb);
        finish(p, r, qa, sa);
        if (++k >= n) break;
        p = pn;
        r = rn;
        if (p != xp) {
            xp = p;
            load_x(p);
        }
        pn = p;
        rn = r + 1;
        if (rn == Rm) {
            rn = 0;
            ++pn;
        }
        const bool more2 = k + 1 < n;
        load(more2 ? pn : p, more2 ? rn : r, qa, sa);
        finish(p, r, qb, sb);
        if (++k >= n) break;
        p = pn;
        r = rn;
        if (p != xp) {
            xp = p;
            load_x(p);
        }
    }
}

// Resident share decoded ahead (the same tasks, plan and arithmetic as
// compute_resident, so the partial sums are bitwise the same): before the
// activation is there, each lane of waves 1..6 decodes its group's tasks
// (at most kOrdPreChunks / UP of them) from the slot into registers, as the
// exact bf16 pairs 16 (c - 8) with the chunk's scale s / 16 beside them; the
// task's part and row go to tpr (p | r << 16).  Once the activation is in
// LDS, dot_predecoded multiplies.
template <int UP>
__device__ __forceinline__ void predecode(const SweepOp& op, const uint8_t* slot, int R, int lane,
                                          uint32_t entry, uint32_t (&wd)[kOrdPreChunks][16],
                                          float (&ws)[kOrdPreChunks], int (&tpr)[kOrdPreChunks]) {
    constexpr int NT = kOrdPreChunks / UP;
    const int n = (int)(entry & 0xFFFFu);
    if (n == 0 || R <= 0) return;
    const int lk = lane & 15;
    const int CP = op.CP, Rm = op.Rm, C = op.C, G = op.G, gshift = op.gshift, rowb = 16 * C;
    const int t0 = (int)(entry >> 16);
    const uint16_t* sslot = reinterpret_cast<const uint16_t*>(slot + kOrdCodeBytes);
    int p = t0 / Rm, r = t0 - p * Rm;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (t < n) {
            tpr[t] = p | (r << 16);
            const int rr = r < R ? r : R - 1;
            const int c0 = p * CP;
#pragma unroll
            for (int u = 0; u < UP; ++u) {
                // chunks past the part's end read the part's first chunk
                // (multiplied by a zero activation)
                const int c = c0 + lk + 16 * u;
                const int cc = c < c0 + CP && c < C ? c : c0;
                const u32x4 q = *reinterpret_cast<const u32x4*>(slot + (size_t)rr * rowb + 16 * cc);
                ws[t * UP + u] = bf16_to_f32(sslot[rr * G + (cc >> gshift)]) * 0.0625f;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const u32x4 v = decode_x16(q[d]);
                    wd[t * UP + u][4 * d + 0] = v[0];
                    wd[t * UP + u][4 * d + 1] = v[1];
                    wd[t * UP + u][4 * d + 2] = v[2];
                    wd[t * UP + u][4 * d + 3] = v[3];
                }
            }
            if (++r == Rm) {
                r = 0;
                ++p;
            }
        }
    }
}

template <int UP>
__device__ __forceinline__ void dot_predecoded(const SweepOp& op, const uint8_t* smem, int R,
                                               int lane, uint32_t entry,
                                               const uint32_t (&wd)[kOrdPreChunks][16],
                                               const float (&ws)[kOrdPreChunks],
                                               const int (&tpr)[kOrdPreChunks]) {
    constexpr int NT = kOrdPreChunks / UP;
    const int n = (int)(entry & 0xFFFFu);
    if (n == 0 || R <= 0) return;
    const int lk = lane & 15;
    const int P = op.P, CP = op.CP, C = op.C;
    float* part = reinterpret_cast<float*>(const_cast<uint8_t*>(smem) + kOutOff);
    uint32_t xr[UP][16];
    int xp = -1;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (t < n) {
            const int p = tpr[t] & 0xFFFF, r = tpr[t] >> 16;
            if (p != xp) {
                xp = p;
#pragma unroll
                for (int u = 0; u < UP; ++u) {
                    const int c0 = p * CP;
                    const int c = c0 + lk + 16 * u;
                    const bool in = c < c0 + CP && c < C;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        u32x4 v = {0u, 0u, 0u, 0u};
                        if (in)
                            v = *reinterpret_cast<const u32x4*>(smem + kXbOff + i * kQStride + 16 * c);
                        xr[u][4 * i + 0] = v[0];
                        xr[u][4 * i + 1] = v[1];
                        xr[u][4 * i + 2] = v[2];
                        xr[u][4 * i + 3] = v[3];
                    }
                }
            }
            // chunk_dot_x16's two chains in its order, then s / 16
            float acc = 0.f;
#pragma unroll
            for (int u = 0; u < UP; ++u) {
                const uint32_t* b = wd[t * UP + u];
                float a0 = 0.f, a1 = 0.f;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    a0 = dot2(b[4 * d + 0], xr[u][4 * d + 0], a0);
                    a1 = dot2(b[4 * d + 1], xr[u][4 * d + 1], a1);
                    a0 = dot2(b[4 * d + 2], xr[u][4 * d + 2], a0);
                    a1 = dot2(b[4 * d + 3], xr[u][4 * d + 3], a1);
                }
                acc = fmaf(ws[t * UP + u], a0 + a1, acc);
            }
            acc = group_sum<16>(acc);
            if (lk == 0 && r < R) part[r * P + p] = acc;
        }
    }
}

// Streamed share (larger than a slot): every wave streams a contiguous part
// of the rows from HBM, the next row group's codes in flight while the
// current one is multiplied; outputs stored at agent scope.
template <int L>
__device__ __forceinline__ void compute_streamed(const SweepOp& op, const uint8_t* smem, int rb,
                                                 int re, int wv, int lane) {
    constexpr int RG = 64 / L;
    const int lk = lane % L, lr = lane / L;
    const int C = op.C, U = op.U;
    const int R = re - rb;
    const int ng = (R + RG - 1) / RG;
    const int g0 = (int)((long long)wv * ng / kOrdWaves);
    const int g1 = (int)((long long)(wv + 1) * ng / kOrdWaves);
    if (g0 >= g1) return;
    uint32_t xr[kPwMaxU][16];
    slice_from_lds<L>(smem, C, U, lk, xr);
    auto load = [&](int g, u32x4 (&q)[kPwMaxU], uint32_t (&sc)[kPwMaxU]) {
        int n = rb + g * RG + lr;
        n = n < re ? n : re - 1;
        const u32x4* cp = op.codes + (size_t)n * C;
        const uint16_t* sp = op.scales + (size_t)n * op.G;
#pragma unroll
        for (int u = 0; u < kPwMaxU; ++u) {
            if (u < U) {
                int c = lk + L * u;
                c = c < C ? c : C - 1;
                q[u] = nt_load(cp + c);
                sc[u] = gload(sp + (c >> op.gshift));
            }
        }
    };
    auto finish = [&](int g, const u32x4 (&q)[kPwMaxU], const uint32_t (&sc)[kPwMaxU]) {
        const float acc = group_sum<L>(row_partial(q, sc, xr, U));
        const int n = rb + g * RG + lr;
        if (lk == 0 && n < re) store_out_agent(op.y, (size_t)n, acc, op.ydt);
    };
    u32x4 qa[kPwMaxU], qb[kPwMaxU];
    uint32_t sa[kPwMaxU], sb[kPwMaxU];
    int g = g0;
    load(g, qa, sa);
    while (true) {
        load(g + 1 < g1 ? g + 1 : g, qb, sb);
        finish(g, qa, sa);
        if (++g >= g1) break;
        load(g + 1 < g1 ? g + 1 : g, qa, sa);
        finish(g, qb, sb);
        if (++g >= g1) break;
    }
    // The last prefetch is still in flight.  Use its registers here, so the
    // compiler waits for it on this path; otherwise it stays pending across
    // the op loop and the compiler waits for it (with vmcnt(0), which also
    // covers the DMA loads of later ops) before the next resident op's
    // compute.
#pragma unroll
    for (int u = 0; u < kPwMaxU; ++u)
        asm volatile("" ::"v"(qa[u]), "v"(qb[u]), "v"(sa[u]), "v"(sb[u]));
}

// The activation slice of a streamed share for gemv_rows: from the
// workgroup's bf16 copy in LDS (the global activation may be stale in this
// CU's L2), converted to fp16 in registers.  The caller has already checked
// that every lane's slice converts exactly (fallback is never reached).
struct LdsX {
    const uint8_t* smem;
    template <int L, int U>
    __device__ __forceinline__ void load(const GemvArgs& a, int lk, uint32_t (&xr)[U][16]) const {
        uint32_t t[kPwMaxU][16];
        slice_from_lds<L, U>(smem, a.C, U, lk, t);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < 16; ++i) xr[u][i] = t[u][i];
    }
    template <int L>
    __device__ __forceinline__ void fallback(const GemvArgs&, int, int, int, int) const {}
};

// Streamed share with L * U == C and an even number of scale groups per row:
// the stand-alone GEMV's fp16 loop (three row groups in flight per wave,
// outputs gathered per 64-row block) over the share's rows, a contiguous part
// per wave, outputs stored at agent scope.
template <int L, int U>
__device__ __forceinline__ void streamed_fast(const SweepOp& op, const uint8_t* smem, int rb,
                                              int re, int wv, int lane) {
    constexpr int RG = 64 / L;
    GemvArgs a;
    a.codes = op.codes + (size_t)rb * op.C;
    a.scales = op.scales + (size_t)rb * op.G;
    a.x = nullptr;
    a.y = static_cast<uint8_t*>(op.y) + (size_t)rb * (op.ydt == W4_BF16 ? 2 : 4);
    a.N = re - rb;
    a.C = op.C;
    a.G = op.G;
    a.gshift = op.gshift;
    a.ydt = op.ydt;
    const int ng = (a.N + RG - 1) / RG;
    const int g0 = (int)((long long)wv * ng / kOrdWaves);
    const int g1 = (int)((long long)(wv + 1) * ng / kOrdWaves);
    if (g0 >= g1) return;
    // a wave with a slice fp16 cannot hold exactly runs the bf16 loop
    {
        uint32_t t[kPwMaxU][16];
        slice_from_lds<L, U>(smem, op.C, U, lane % L, t);
        u16x2 mx = {0, 0}, mn = {0xFFFF, 0xFFFF};
#pragma unroll
        for (int u = 0; u < U; ++u) pairs_range(t[u], 16, mx, mn);
        bool ok = true;
        (void)f16_scale_exp(mx, mn, ok);
        if (wave_any_inexact(ok)) {
            compute_streamed<L>(op, smem, rb, re, wv, lane);
            return;
        }
    }
    const DecodeConsts k = decode_consts();
    gemv_rows<L, U, true, 3, true, true>(a, g0, g1, 1, lane, k, LdsX{smem});
}

// A streamed share, every wave of the workgroup; its outputs are stored and
// complete when it returns.  (The wait sits on this path itself, so that the
// compiler knows no load of it is still in flight afterwards.)
__device__ __forceinline__ void compute_streamed_op(const SweepOp& op, const uint8_t* smem,
                                                    int rb, int re, int wave, int lane) {
    bool done = false;
    if (op.L * op.U == op.C && (op.G & 1) == 0) {
        done = true;
        switch (op.L * 8 + op.U) {
            case 16 * 8 + 3: streamed_fast<16, 3>(op, smem, rb, re, wave, lane); break;
            case 16 * 8 + 4: streamed_fast<16, 4>(op, smem, rb, re, wave, lane); break;
            case 32 * 8 + 3: streamed_fast<32, 3>(op, smem, rb, re, wave, lane); break;
            case 32 * 8 + 4: streamed_fast<32, 4>(op, smem, rb, re, wave, lane); break;
            case 64 * 8 + 3: streamed_fast<64, 3>(op, smem, rb, re, wave, lane); break;
            case 64 * 8 + 4: streamed_fast<64, 4>(op, smem, rb, re, wave, lane); break;
            default: done = false; break;
        }
    }
    if (!done) {
        switch (op.L) {
            case 16: compute_streamed<16>(op, smem, rb, re, wave, lane); break;
            case 32: compute_streamed<32>(op, smem, rb, re, wave, lane); break;
            default: compute_streamed<64>(op, smem, rb, re, wave, lane); break;
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
}

// State of one workgroup across the ops of a replay.
struct OrdCtx {
    const SweepOp* ops;
    SweepCtl* ctl;
    uint8_t* smem;
    int* s_flags;   // [i & 1] op i may run; [2] compute-wave completions; [3] (pre) slot landed
    int w, G, wave, lane;
    // DMA loads issued after those of the next resident op
    int pend_next;
    // the resident op whose share is DMA'd next (see ordered_kernel)
    SweepOp nx;
    int nx_slot;
    // running count of compute-wave completions wave 0 waits for
    unsigned arrived;
    // (pre) ops below this index have been flagged as landed
    int landed;
    // completion polls per op before giving up
    unsigned poll_limit;
    __device__ uint8_t* slot_at(int sl) const { return smem + sl * kSlotBytes; }
};

// Wave 0: wait until every workgroup has signalled op i - 1 (or the error
// word is set), publish the verdict for op i in LDS and, if op i may run,
// load its activation into LDS.  One poll in flight at a time: more (four,
// 130 ns apart) measured slower, the extra reads of the counters' lines
// slowing the signals themselves (547 against 537 us per step).
__device__ __forceinline__ void handoff_in(OrdCtx& k, const SweepOp& op, int i) {
    bool ok = true;
    if (i > 0) {
        ok = false;
        // lanes 0..7 read the counters, lane 8 the error word (the others
        // re-read counter 0 and are ignored)
        const unsigned* p = k.lane < 8 ? &k.ctl->cnt[32 * k.lane]
                                       : (k.lane == 8 ? &k.ctl->error : &k.ctl->cnt[0]);
        const unsigned target = (unsigned)i * (unsigned)k.G;
        for (unsigned spin = 0; spin < k.poll_limit; ++spin) {
            const unsigned v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            // lanes 0..7 summed and lane 8's word, read into scalar registers
            unsigned c = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) c += __builtin_amdgcn_readlane(v, j);
            const unsigned e = __builtin_amdgcn_readlane(v, 8);
            if ((int)(c - target) >= 0) {
                ok = true;
                break;
            }
            if (e) break;
        }
    }
    if (k.lane == 0) {
        if (!ok) __hip_atomic_store(&k.ctl->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        k.s_flags[i & 1] = ok ? 1 : 0;
    }
    if (ok) load_x_dma(op.x, op.C, k.lane, k.smem);
    wait_vm<0>();   // the activation has landed
}

// After the compute: the compute waves (0..6 for a resident share, all 8
// for a streamed one) count themselves done in LDS, partial sums written
// (resident) or outputs stored and complete (streamed); wave 0 waits for the
// count (not a workgroup barrier, so the DMA wave, whose copy may still be
// issuing, holds nobody up), adds a resident share's partial sums, stores
// the outputs, waits for them to complete and signals.
__device__ __forceinline__ void handoff_out(OrdCtx& k, const SweepOp& op, int rb, int re) {
    const bool computes = !op.res || k.wave != kOrdDmaWave;
    k.arrived += op.res ? kOrdWaves - 1 : kOrdWaves;
    if (computes && k.lane == 0)
        __hip_atomic_fetch_add(&k.s_flags[2], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (k.wave != 0) return;
    // a tight spin (no sleep between the LDS reads: 3 us less per step)
    bool done = false;
    for (unsigned spin = 0; spin < kOrdSpin; ++spin) {
        const unsigned c = (unsigned)__hip_atomic_load(&k.s_flags[2], __ATOMIC_ACQUIRE,
                                                       __HIP_MEMORY_SCOPE_WORKGROUP);
        if ((int)(c - k.arrived) >= 0) {
            done = true;
            break;
        }
    }
    if (!done) {
        // cannot happen unless a wave is lost; the next poll sees the error
        // word and every workgroup leaves
        if (k.lane == 0)
            __hip_atomic_store(&k.ctl->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    if (op.res) {
        // a row's P partial sums, added in order
        const float* part = reinterpret_cast<const float*>(k.smem + kOutOff);
        for (int r = k.lane; r < re - rb; r += 64) {
            float v = part[r * op.P];
            for (int q = 1; q < op.P; ++q) v += part[r * op.P + q];
            store_out_agent(op.y, (size_t)(rb + r), v, op.ydt);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);   // the outputs are visible to every CU
    asm volatile("" ::: "memory");
    if (k.lane == 0)
        __hip_atomic_fetch_add(&k.ctl->cnt[32 * (k.w & 7)], 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
}

// One op decoded in the compute (streamed shares; resident shares unless
// decoded ahead).  Returns false when the workgroup is to leave.
__device__ __forceinline__ bool inline_op(OrdCtx& k, const SweepOp& op, int i, uint32_t entry) {
    int rb, re;
    share_rows(op.N, k.w, k.G, rb, re);
    if (k.wave == kOrdDmaWave && op.res) {
        // this op's share has landed once only the DMA loads issued after it
        // are in flight
        wait_vm_rt(k.pend_next);
        k.pend_next = 0;
    }
    if (k.wave == 0) handoff_in(k, op, i);
    __syncthreads();   // A: the verdict, the activation and the weights of op i
    if (k.s_flags[i & 1] == 0) return false;
    if (k.wave == kOrdDmaWave && op.res && k.nx_slot >= 0) {
        // the previous resident op's slot is free: the resident op after this
        // one goes in.  Issued here, not when that slot was freed, so that
        // the DMA traffic overlaps this op's compute (which reads only LDS)
        // instead of the handoff's stores, polls and loads.
        issue_share(k.nx, k.w, k.G, k.slot_at(k.nx_slot), k.lane);
        k.nx_slot = -1;
    }
    if (op.res) {
        if (k.wave < kOrdDmaWave) {
            const uint8_t* slot = k.slot_at(op.slot);
            const int R = re - rb;
            switch (op.UP) {
                case 1: compute_resident<1>(op, k.smem, slot, R, k.lane, entry); break;
                case 2: compute_resident<2>(op, k.smem, slot, R, k.lane, entry); break;
                case 3: compute_resident<3>(op, k.smem, slot, R, k.lane, entry); break;
                default: compute_resident<4>(op, k.smem, slot, R, k.lane, entry); break;
            }
        }
    } else {
        compute_streamed_op(op, k.smem, rb, re, k.wave, k.lane);
    }
    handoff_out(k, op, rb, re);
    if (k.wave == kOrdDmaWave && op.res && op.next >= 0) {
        // the slot is free once the compute waves are past this op (they are
        // when the next op's barrier A opens): the resident op after the
        // next one goes in once the next resident op starts computing
        k.nx = k.ops[op.next];
        k.nx_slot = k.nx.slot;
    }
    return true;
}

// DMA wave: resident op i's share is in LDS (its DMA loads have been
// waited for).  A relaxed store after that explicit wait: a release store
// would also wait for every other DMA load in flight.
__device__ __forceinline__ void flag_landed(OrdCtx& k, int i) {
    asm volatile("" ::: "memory");
    if (k.lane == 0)
        __hip_atomic_store(&k.s_flags[3], i + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    k.landed = i + 1;
}

// One resident op decoded ahead: the DMA wave flags the share as landed;
// waves 1..6 decode their tasks into registers while wave 0 waits for op
// i - 1 and loads the activation; after barrier A the DMA wave sends op i's
// successor-but-one into op i's slot (already decoded) and waves 1..6
// multiply.  Returns false when the workgroup is to leave.
template <int UP>
__device__ __forceinline__ bool predecoded_op(OrdCtx& k, const SweepOp& op, int i,
                                              uint32_t entry) {
    int rb, re;
    share_rows(op.N, k.w, k.G, rb, re);
    const int R = re - rb;
    uint32_t wd[kOrdPreChunks][16];
    float ws[kOrdPreChunks];
    int tpr[kOrdPreChunks];
    if (k.wave == kOrdDmaWave) {
        if (k.landed <= i) {
            // the first resident op: its share is in LDS once only the DMA
            // loads issued after it are in flight (later ones are flagged at
            // the previous resident op's barrier A)
            wait_vm_rt(k.pend_next);
            k.pend_next = 0;
            flag_landed(k, i);
        }
        if (op.next >= 0) k.nx = k.ops[op.next];
    } else if (k.wave != 0) {
        bool landed = false;
        for (unsigned spin = 0; spin < kOrdSpin; ++spin) {
            if (__hip_atomic_load(&k.s_flags[3], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) > i) {
                landed = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (landed) {
            predecode<UP>(op, k.slot_at(op.slot), R, k.lane, entry, wd, ws, tpr);
        } else if (k.lane == 0) {
            // cannot happen unless the DMA wave is lost; the next poll sees
            // the error word and every workgroup leaves
            __hip_atomic_store(&k.ctl->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    } else {
        handoff_in(k, op, i);
    }
    __syncthreads();   // A: the verdict and the activation of op i; op i's slot decoded
    if (k.s_flags[i & 1] == 0) return false;
    if (k.wave == kOrdDmaWave) {
        // the next resident op's share, the only DMA in flight (issued at the
        // previous barrier A), is flagged as soon as it has landed, so that
        // its decode can start when this op's multiply ends; then the
        // resident op after it goes into this op's slot (already decoded)
        if (op.nres >= 0) {
            wait_vm<0>();
            flag_landed(k, op.nres);
        }
        if (op.next >= 0) issue_share(k.nx, k.w, k.G, k.slot_at(op.slot), k.lane);
    } else if (k.wave != 0) {
        dot_predecoded<UP>(op, k.smem, R, k.lane, entry, wd, ws, tpr);
    }
    handoff_out(k, op, rb, re);
    return true;
}

}  // namespace

// pre: every resident op's share is decoded ahead (predecoded_op); the
// host's plans then give wave 0 no tasks.
__global__ __launch_bounds__(kOrdThreads) void ordered_kernel(const SweepOp* __restrict__ ops,
                                                              int n_ops, SweepCtl* ctl,
                                                              int first0, int first1, int pre,
                                                              unsigned poll_limit) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x;
    OrdCtx k;
    k.ops = ops;
    k.ctl = ctl;
    k.smem = smem;
    k.s_flags = reinterpret_cast<int*>(smem + kFlagOff);
    k.lane = tid & 63;
    k.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    k.G = gridDim.x;
    k.w = blockIdx.x;
    k.nx_slot = -1;
    k.arrived = 0;
    k.landed = 0;
    k.poll_limit = poll_limit;
    if (tid == 0) {
        k.s_flags[2] = 0;
        k.s_flags[3] = 0;
    }
    __syncthreads();

    // the first two resident ops' shares go to the slots at once
    if (k.wave == kOrdDmaWave) {
        if (first0 >= 0) issue_share(ops[first0], k.w, k.G, k.slot_at(ops[first0].slot), k.lane);
        if (first1 >= 0) issue_share(ops[first1], k.w, k.G, k.slot_at(ops[first1].slot), k.lane);
    }
    k.pend_next = first1 >= 0 ? share_dmas(ops[first1], k.w, k.G) : 0;
    // this lane's group's task run of the next op, read one op ahead so that
    // the load's latency hides behind the current op (a global-typed load:
    // a generic one would also hold the LDS counter)
    uint32_t entry_next = 0;
    if (ops[0].res && k.wave < kOrdDmaWave)
        entry_next = gload(ops[0].plan + 4 * k.wave + (k.lane >> 4));

    for (int i = 0; i < n_ops; ++i) {
        const SweepOp op = ops[i];
        const uint32_t entry = entry_next;
        if (i + 1 < n_ops && k.wave < kOrdDmaWave && ops[i + 1].res)
            entry_next = gload(ops[i + 1].plan + 4 * k.wave + (k.lane >> 4));
        bool go;
        if (pre && op.res) {
            switch (op.UP) {
                case 1: go = predecoded_op<1>(k, op, i, entry); break;
                case 2: go = predecoded_op<2>(k, op, i, entry); break;
                case 3: go = predecoded_op<3>(k, op, i, entry); break;
                default: go = predecoded_op<4>(k, op, i, entry); break;
            }
        } else {
            go = inline_op(k, op, i, entry);
        }
        if (!go) {
            __builtin_amdgcn_s_waitcnt(0);   // no DMA into LDS outlives the workgroup
            return;
        }
    }

    // the last workgroup to finish resets the counters for the next replay;
    // every access of this workgroup (its last signal included) completes
    // before it counts itself finished
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
    if (tid == 0) {
        const unsigned done = __hip_atomic_fetch_add(&ctl->fin, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (done == (unsigned)k.G - 1u) {
#pragma unroll
            for (int x = 0; x < 8; ++x)
                __hip_atomic_store(&ctl->cnt[32 * x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&ctl->fin, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

int ordered_lds_bytes() { return kOrdLds; }

}  // namespace w4
