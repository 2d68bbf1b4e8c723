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
//  - weights never depend on activations: waves 1..7 DMA the workgroup's
//    share of the next resident op (codes and scales, up to 56 KB) into one
//    of two LDS slots while the current op waits and computes, so an op's
//    compute reads its weights from LDS;
//  - wave 0 is the control wave: it issues no DMA (so its waits cover only
//    its own accesses), polls the completion counters, loads the activation
//    (agent scope, 16-byte loads) into LDS for the whole workgroup, stores
//    the workgroup's outputs (agent scope), waits for them to complete and
//    signals;
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
constexpr int kOutOff = kXbOff + kOrdMaxK * 2;          // the share's outputs (fp32)
constexpr int kFlagOff = kOutOff + kOrdMaxRows * 4;     // s_ok
constexpr int kOrdLds = kFlagOff + 16;

__device__ __forceinline__ void share_rows(int N, int w, int G, int& rb, int& re) {
    rb = (int)((long long)w * N / G);
    re = (int)((long long)(w + 1) * N / G);
}

// wait until at most n of this wave's DMA loads are in flight (0 <= n < 64)
__device__ __forceinline__ void wait_vm_rt(int n) {
    switch (n) {
#define W4_CASE(N) case N: wait_vm<N>(); break;
        W4_CASE(0) W4_CASE(1) W4_CASE(2) W4_CASE(3) W4_CASE(4) W4_CASE(5) W4_CASE(6)
        W4_CASE(7) W4_CASE(8) W4_CASE(9) W4_CASE(10) W4_CASE(11) W4_CASE(12) W4_CASE(13)
        W4_CASE(14) W4_CASE(15) W4_CASE(16)
#undef W4_CASE
        default: wait_vm<0>(); break;
    }
}

// DMA instructions each DMA wave issues for a share of `bytes` bytes (1 KB
// per wave per instruction, waves 1..7 side by side).
__device__ __forceinline__ int dma_rounds(int bytes) {
    return (bytes + kOrdDmaWaves * 1024 - 1) / (kOrdDmaWaves * 1024);
}

// Issue the DMA of op's share for workgroup w into `slot` (DMA wave dw =
// 0..6).  Codes [rb K/2, re K/2) and scales [rb G 2, re G 2) are contiguous
// byte ranges, whole 16-byte units for a resident op (K % 256 == 0 and
// G % 8 == 0, checked on the host); lanes past a range re-read its last 16
// bytes into slot space past the share.  An empty share issues nothing.
__device__ __forceinline__ void issue_share(const SweepOp& op, int w, int G, uint8_t* slot,
                                            int dw, int lane) {
    int rb, re;
    share_rows(op.N, w, G, rb, re);
    const int K = op.C * 32;
    const uint32_t cb = (uint32_t)(re - rb) * (uint32_t)(K / 2);
    const uint32_t c0 = (uint32_t)rb * (uint32_t)(K / 2);
    const int nc = dma_rounds((int)cb);
    const uint32_t lds0 = lds_addr(slot);
    for (int d = 0; d < nc; ++d) {
        const uint32_t o = (uint32_t)(d * kOrdDmaWaves + dw) * 1024u + 16u * lane;
        const uint32_t src = c0 + (o < cb ? o : (cb >= 16u ? cb - 16u : 0u));
        dma16(src, op.codes, lds0 + (uint32_t)(d * kOrdDmaWaves + dw) * 1024u);
    }
    const uint32_t sb = (uint32_t)(re - rb) * (uint32_t)(op.G * 2);
    const uint32_t s0 = (uint32_t)rb * (uint32_t)(op.G * 2);
    const int ns = dma_rounds((int)sb);
    for (int d = 0; d < ns; ++d) {
        const uint32_t o = (uint32_t)(d * kOrdDmaWaves + dw) * 1024u + 16u * lane;
        const uint32_t src = s0 + (o < sb ? o : (sb >= 16u ? sb - 16u : 0u));
        dma16(src, op.scales, lds0 + kOrdCodeBytes + (uint32_t)(d * kOrdDmaWaves + dw) * 1024u);
    }
}

__device__ __forceinline__ int share_dmas(const SweepOp& op, int w, int G) {
    int rb, re;
    share_rows(op.N, w, G, rb, re);
    return dma_rounds((re - rb) * (op.C * 16)) + dma_rounds((re - rb) * (op.G * 2));
}

// Chunks c0 + 64 j (j = 0..3) of an activation as agent-scope 16-byte loads
// (written by any CU; sc1 loads are coherent across XCDs, as the
// compiler's own agent-scope loads are), all in flight at once; chunks at or
// past C re-read chunk C - 1.  The caller has no other vector-memory access
// in flight that it needs to overlap (one wait covers everything).
__device__ __forceinline__ void load_x4_agent(const uint32_t* x, int c0, int C,
                                              u32x4 (&v)[4][4]) {
    const uint8_t* p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = c0 + 64 * j < C ? c0 + 64 * j : C - 1;
        p[j] = reinterpret_cast<const uint8_t*>(x + 16 * c);
    }
    asm volatile(
        "global_load_dwordx4 %0, %16, off sc1\n\t"
        "global_load_dwordx4 %1, %16, off offset:16 sc1\n\t"
        "global_load_dwordx4 %2, %16, off offset:32 sc1\n\t"
        "global_load_dwordx4 %3, %16, off offset:48 sc1\n\t"
        "global_load_dwordx4 %4, %17, off sc1\n\t"
        "global_load_dwordx4 %5, %17, off offset:16 sc1\n\t"
        "global_load_dwordx4 %6, %17, off offset:32 sc1\n\t"
        "global_load_dwordx4 %7, %17, off offset:48 sc1\n\t"
        "global_load_dwordx4 %8, %18, off sc1\n\t"
        "global_load_dwordx4 %9, %18, off offset:16 sc1\n\t"
        "global_load_dwordx4 %10, %18, off offset:32 sc1\n\t"
        "global_load_dwordx4 %11, %18, off offset:48 sc1\n\t"
        "global_load_dwordx4 %12, %19, off sc1\n\t"
        "global_load_dwordx4 %13, %19, off offset:16 sc1\n\t"
        "global_load_dwordx4 %14, %19, off offset:32 sc1\n\t"
        "global_load_dwordx4 %15, %19, off offset:48 sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[0][2]), "=&v"(v[0][3]), "=&v"(v[1][0]),
          "=&v"(v[1][1]), "=&v"(v[1][2]), "=&v"(v[1][3]), "=&v"(v[2][0]), "=&v"(v[2][1]),
          "=&v"(v[2][2]), "=&v"(v[2][3]), "=&v"(v[3][0]), "=&v"(v[3][1]), "=&v"(v[3][2]),
          "=&v"(v[3][3])
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3])
        : "memory");
}

// One lane's activation slice for tile (L, U): chunks chunk_of(lk, rot, u)
// of the workgroup's bf16 copy in LDS; chunks past the row end read as zero.
// The lanes of a row take its chunks (lk + rot) mod L + L u: a row's lanes
// still cover every chunk, and with rot = 4 (row within the wave) the rows a
// wave reads at once start on different LDS banks.
template <int L>
__device__ __forceinline__ int chunk_of(int lk, int rot, int u) {
    return ((lk + rot) & (L - 1)) + L * u;
}

// UT > 0: the chunk count U per lane is the compile-time UT (every load can
// be issued up front); UT == 0: U at run time.
template <int L, int UT = 0>
__device__ __forceinline__ void slice_from_lds(const uint8_t* smem, int C, int U, int lk, int rot,
                                               uint32_t (&xr)[kPwMaxU][16]) {
#pragma unroll
    for (int u = 0; u < (UT > 0 ? UT : kPwMaxU); ++u) {
        const int c = chunk_of<L>(lk, rot, u);
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

// Resident share: rows 0 .. R-1 of the slot, row groups of 64/L rows taken by
// the workgroup's 8 waves in turn; row sums go to the LDS output buffer.
template <int L, int UT = 0>
__device__ __forceinline__ void compute_resident(const SweepOp& op, const uint8_t* smem,
                                                 const uint8_t* slot, int R, int wave,
                                                 int lane) {
    constexpr int RG = 64 / L;
    const int lk = lane % L, lr = lane / L;
    const int C = op.C, U = UT > 0 ? UT : op.U, K = C * 32;
    const int ngroups = (R + RG - 1) / RG;
    if (wave >= ngroups) return;
    const int rot = 4 * lr;
    uint32_t xr[kPwMaxU][16];
    slice_from_lds<L, UT>(smem, C, U, lk, rot, xr);
    float* outv = reinterpret_cast<float*>(const_cast<uint8_t*>(smem) + kOutOff);
    const uint16_t* sslot = reinterpret_cast<const uint16_t*>(slot + kOrdCodeBytes);
    for (int g = wave; g < ngroups; g += kOrdWaves) {
        int r = g * RG + lr;
        const bool live = r < R;
        r = live ? r : R - 1;
        u32x4 q[kPwMaxU];
        uint32_t sc[kPwMaxU];
#pragma unroll
        for (int u = 0; u < (UT > 0 ? UT : kPwMaxU); ++u) {
            int c = chunk_of<L>(lk, rot, u);
            c = c < C ? c : C - 1;
            q[u] = *reinterpret_cast<const u32x4*>(slot + (size_t)r * (K / 2) + 16 * c);
            sc[u] = sslot[r * op.G + (c >> op.gshift)];
        }
        const float acc = group_sum<L>(row_partial<UT>(q, sc, xr, U));
        if (lk == 0 && live) outv[r] = acc;
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
    slice_from_lds<L>(smem, C, U, lk, 0, xr);
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
    __device__ __forceinline__ bool load(const GemvArgs& a, int lk, uint32_t (&xr)[U][16],
                                         float& xv) const {
        uint32_t t[kPwMaxU][16];
        slice_from_lds<L, U>(smem, a.C, U, lk, 0, t);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < 16; ++i) xr[u][i] = t[u][i];
        bool ok = true;
        xv = chunks_to_f16<U>(xr, ok);
        return ok;
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
        slice_from_lds<L, U>(smem, op.C, U, lane % L, 0, t);
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

__device__ __forceinline__ void compute_op(const SweepOp& op, const uint8_t* smem,
                                           const uint8_t* slot, int rb, int re, int wave,
                                           int lane) {
    if (op.res) {
        const int R = re - rb;
        // the lane tilings of the ordered sweep (L from the row length,
        // U = ceil(C / L)) with U known at compile time
        switch (op.L * 8 + op.U) {
            case 16 * 8 + 1: compute_resident<16, 1>(op, smem, slot, R, wave, lane); return;
            case 16 * 8 + 2: compute_resident<16, 2>(op, smem, slot, R, wave, lane); return;
            case 16 * 8 + 3: compute_resident<16, 3>(op, smem, slot, R, wave, lane); return;
            case 16 * 8 + 4: compute_resident<16, 4>(op, smem, slot, R, wave, lane); return;
            case 32 * 8 + 3: compute_resident<32, 3>(op, smem, slot, R, wave, lane); return;
            case 32 * 8 + 4: compute_resident<32, 4>(op, smem, slot, R, wave, lane); return;
            case 64 * 8 + 3: compute_resident<64, 3>(op, smem, slot, R, wave, lane); return;
            case 64 * 8 + 4: compute_resident<64, 4>(op, smem, slot, R, wave, lane); return;
            default: break;
        }
        switch (op.L) {
            case 16: compute_resident<16>(op, smem, slot, R, wave, lane); break;
            case 32: compute_resident<32>(op, smem, slot, R, wave, lane); break;
            default: compute_resident<64>(op, smem, slot, R, wave, lane); break;
        }
    } else {
        if (op.L * op.U == op.C && (op.G & 1) == 0) {
            switch (op.L * 8 + op.U) {
                case 16 * 8 + 3: streamed_fast<16, 3>(op, smem, rb, re, wave, lane); return;
                case 16 * 8 + 4: streamed_fast<16, 4>(op, smem, rb, re, wave, lane); return;
                case 32 * 8 + 3: streamed_fast<32, 3>(op, smem, rb, re, wave, lane); return;
                case 32 * 8 + 4: streamed_fast<32, 4>(op, smem, rb, re, wave, lane); return;
                case 64 * 8 + 3: streamed_fast<64, 3>(op, smem, rb, re, wave, lane); return;
                case 64 * 8 + 4: streamed_fast<64, 4>(op, smem, rb, re, wave, lane); return;
                default: break;
            }
        }
        switch (op.L) {
            case 16: compute_streamed<16>(op, smem, rb, re, wave, lane); break;
            case 32: compute_streamed<32>(op, smem, rb, re, wave, lane); break;
            default: compute_streamed<64>(op, smem, rb, re, wave, lane); break;
        }
    }
}

}  // namespace

__global__ __launch_bounds__(kOrdThreads) void ordered_kernel(const SweepOp* __restrict__ ops,
                                                              int n_ops, SweepCtl* ctl,
                                                              int first0, int first1) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = gridDim.x;
    const int w = blockIdx.x;
    int* s_flags = reinterpret_cast<int*>(smem + kFlagOff);   // [0] ok
    auto slot_at = [&](int sl) { return smem + sl * kSlotBytes; };

    // the first two resident ops' shares go to the slots at once
    if (wave > 0) {
        if (first0 >= 0) issue_share(ops[first0], w, G, slot_at(ops[first0].slot), wave - 1, lane);
        if (first1 >= 0) issue_share(ops[first1], w, G, slot_at(ops[first1].slot), wave - 1, lane);
    }
    // DMA loads this wave has issued and not yet waited for, per pending op
    int pend_next = first1 >= 0 ? share_dmas(ops[first1], w, G) : 0;

    for (int i = 0; i < n_ops; ++i) {
        const SweepOp op = ops[i];
        int rb, re;
        share_rows(op.N, w, G, rb, re);

        if (wave == 0) {
            // wait for op i-1 (every workgroup has signalled it)
            bool ok = true;
            if (i > 0) {
                ok = false;
                const unsigned target = (unsigned)i * (unsigned)G;
                for (unsigned spin = 0; spin < kOrdSpin; ++spin) {
                    // one round trip per poll: lanes 0..7 read the counters,
                    // lane 8 the error word
                    unsigned c = 0, e = 0;
                    if (lane < 8)
                        c = __hip_atomic_load(&ctl->cnt[32 * lane], __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
                    else if (lane == 8)
                        e = __hip_atomic_load(&ctl->error, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
                    c += __shfl_xor(c, 1, 64);
                    c += __shfl_xor(c, 2, 64);
                    c += __shfl_xor(c, 4, 64);
                    c = __shfl(c, 0, 64);   // lane 0's total on every lane
                    e = __shfl(e, 8, 64);
                    if ((int)(c - target) >= 0) {
                        ok = true;
                        break;
                    }
                    if (e) break;
                }
            }
            // op i's activation (written by any CU): agent-scope loads into
            // the workgroup's bf16 copy
            if (ok && lane < op.C) {
                u32x4 xg[4][4];
                load_x4_agent(reinterpret_cast<const uint32_t*>(op.x), lane, op.C, xg);
                uint32_t* xb = reinterpret_cast<uint32_t*>(smem + kXbOff);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = lane + 64 * j;
                    if (c < op.C) {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            *reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(xb) +
                                                      q * kQStride + 16 * c) = xg[j][q];
                    }
                }
            }
            if (lane == 0) {
                if (!ok)
                    __hip_atomic_store(&ctl->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                s_flags[0] = ok ? 1 : 0;
            }
        }
        if (wave > 0 && op.res) {
            // this op's share has landed: only the next resident op's DMA
            // loads may still be in flight
            wait_vm_rt(pend_next);
        }
        __syncthreads();   // A: activation and weights of op i visible
        if (s_flags[0] == 0) {
            __builtin_amdgcn_s_waitcnt(0);   // no DMA into LDS outlives the workgroup
            return;
        }
        const uint8_t* slot = slot_at(op.slot);
        compute_op(op, smem, slot, rb, re, wave, lane);
        if (!op.res) {
            // streamed outputs were stored by every wave: complete before B
            __builtin_amdgcn_s_waitcnt(0);
            asm volatile("" ::: "memory");
        }
        __syncthreads();   // B: every output of the share computed (and stored)

        if (wave == 0) {
            if (op.res) {
                const float* outv = reinterpret_cast<const float*>(smem + kOutOff);
                for (int r = lane; r < re - rb; r += 64)
                    store_out_agent(op.y, (size_t)(rb + r), outv[r], op.ydt);
            }
            __builtin_amdgcn_s_waitcnt(0);   // the outputs are visible to every CU
            asm volatile("" ::: "memory");
            if (lane == 0)
                __hip_atomic_fetch_add(&ctl->cnt[32 * (w & 7)], 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        } else if (op.res) {
            // the slot is free: the resident op after the next one goes in
            if (op.next >= 0) {
                const SweepOp nx = ops[op.next];
                issue_share(nx, w, G, slot_at(nx.slot), wave - 1, lane);
                // pending now: the next resident op's loads, then these
                const int mine = share_dmas(nx, w, G);
                pend_next = mine;
            } else {
                pend_next = 0;
            }
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
        if (done == (unsigned)G - 1u) {
#pragma unroll
            for (int x = 0; x < 8; ++x)
                __hip_atomic_store(&ctl->cnt[32 * x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&ctl->fin, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

int ordered_lds_bytes() { return kOrdLds; }

}  // namespace w4
