// w4_gemv_core.h -- the batch-1 GEMV inner loop, shared by the stand-alone
// GEMV kernel and the persistent decode-step kernel (internal).
//
// [P1] "Gemma 4 E2B on a 4 GB GPU with plain PyTorch, faster than llama.cpp",
// paragraph on the w4gemv.py kernel: packed 4-bit words are read once,
// unpacked in registers and multiplied; a fixed tiling per weight shape.
//
// A row of K codes is C = K/32 chunks of 16 bytes (32 codes, one dwordx4
// load, one K-group of 32).  L lanes share a row; lane l of a row owns chunks
// l, l + L, ..., l + (U-1)L, so for each u the L lanes read L consecutive
// chunks and a wave reads R = 64/L rows at once (a "row group").  A lane's
// chunks are the same for every row, so its activation slice stays in
// registers, converted once to fp16 with one power-of-two scale per lane
// (w4_common.h); the codes are decoded to the exact fp16 values c - 8.  A
// wave with a lane whose slice fp16 cannot represent exactly (a dynamic
// range beyond 2^29, inf or NaN) runs the exact bf16 loop instead.
#pragma once

#include "w4_dispatch.h"

namespace w4 {

struct GemvArgs {
    const u32x4* codes;      // N x C chunks (device words)
    const uint16_t* scales;  // N x G bf16
    const uint32_t* x;       // K/2 bf16 pairs
    void* y;
    int N, C, G, gshift, ydt;
};

// Issues the loads of this lane's activation slice (bf16 pairs; zero slices
// for chunks past the row end).  x_slice_to_f16 converts it once it is in.
template <int L, int U>
__device__ __forceinline__ void load_x_slice(const uint32_t* x, int C, int lk,
                                             uint32_t (&xr)[U][16]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = lk + L * u;
        if (c < C) {
            const u32x4* p = reinterpret_cast<const u32x4*>(x + 16 * c);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x4 v = gload(p + i);
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

// Converts a lane's activation slice to fp16 pairs in place and sets xv to
// its inverse scale; returns whether the conversion was exact.
template <int U>
__device__ __forceinline__ bool x_slice_to_f16(uint32_t (&xr)[U][16], float& xv) {
    bool ok = true;
    xv = chunks_to_f16<U>(xr, ok);
    return ok;
}

// True when some lane of the wave saw a chunk fp16 cannot hold exactly.
__device__ __forceinline__ bool wave_any_inexact(bool ok) {
    return __builtin_amdgcn_ballot_w64(!ok) != 0;
}

template <int L>
__device__ __forceinline__ void gemv_rows_generic(const struct GemvArgs& a, int rg0, int rg1,
                                                  int step, int lane);

// Where gemv_rows takes a lane's activation slice from, and what it runs when
// the slice is not exact in fp16.  GlobalX: the slice from a.x in global
// memory (written before the launch), the exact bf16 loop as fallback.
struct GlobalX {
    template <int L, int U>
    __device__ __forceinline__ void load(const GemvArgs& a, int lk, uint32_t (&xr)[U][16]) const {
        load_x_slice<L, U>(a.x, a.C, lk, xr);
    }
    template <int L>
    __device__ __forceinline__ void fallback(const GemvArgs& a, int rg0, int rg1, int step,
                                             int lane) const {
        gemv_rows_generic<L>(a, rg0, rg1, step, lane);
    }
};

// Row groups rg0, rg0 + step, ... (< rg1) of one matrix for one wave.
// Needs an even number of groups per row (G).  FULLC: L * U == C.  Otherwise lanes past the row end read a clamped, valid
// chunk and multiply it by a zero activation slice.  Rows past N are clamped
// to row N - 1 and not stored, so the loop has no divergent branches.
// XS supplies the activation slice and the exact fallback (GlobalX); AGENT
// stores the outputs at agent scope (read by other CUs in the same launch).
// STAGES register sets rotate: STAGES - 1 row groups are in flight while the
// current one is decoded.  Lane partials are summed in a fixed order, so the
// result is bitwise deterministic.
// BATCH (consecutive row groups, step == 1): outputs are gathered into one
// register and each 64-row block is written with one store when the walk
// leaves it (128 or 256 contiguous bytes instead of a few bytes per row
// group: small scattered writes in a stream of reads cost HBM read
// bandwidth).  Lane l holds row R * (l % L) + l / L of the block, i.e. row r
// of the block's row group t sits in lane L r + t: after the 16-lane DPP row
// sums every lane of a 16-lane row already holds its row's total, so a row
// group's outputs are taken with one compare and no cross-lane move (32- and
// 64-lane rows finish with DPP row broadcasts and one readlane per row).
template <int L, int U, bool FULLC, int STAGES = 2, bool BATCH = false, bool AGENT = false,
          class XS = GlobalX>
__device__ __forceinline__ void gemv_rows(const GemvArgs& a, int rg0, int rg1, int step,
                                          int lane, const DecodeConsts& k, const XS& xs = XS()) {
    static_assert(STAGES == 2 || STAGES == 3, "register stages");
    constexpr int R = 64 / L;
    if (rg0 >= rg1) return;
    // lane-derived offsets are formed per call, not hoisted to the kernel's
    // entry (a kernel with several tile shapes would hold all of them live)
    asm volatile("" : "+v"(lane));
    const int lk = lane % L;
    const int lr = lane / L;

    // the activation slice's loads go first, then (below) the first row
    // groups' codes; the conversion waits for the slice only
    uint32_t xr[U][16];
    float xv;
    xs.template load<L, U>(a, lk, xr);

    // chunk offsets, scale dword offsets and scale half selectors per chunk
    int coff[U], soff[U];
    uint32_t ssel[U];
    const int sbase = (lk >> a.gshift) >> 1;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int c = lk + L * u;
        if (!FULLC && c >= a.C) c = a.C - 1;
        const int cg = c >> a.gshift;
        coff[u] = c - lk;
        soff[u] = (cg >> 1) - sbase;
        ssel[u] = (cg & 1) ? kScaleSelHi : kScaleSelLo;
    }
    const uint32_t* swords = reinterpret_cast<const uint32_t*>(a.scales);
    const int Gw = a.G >> 1;

    float outv = 0.f;               // BATCH: lane l = row ob + R (l % L) + l / L
    int ob = -1, olo = 0, ohi = 0;  // block base row, row groups written so far
    auto flush = [&]() {
        const int t = lane % L;
        const int n = ob + R * t + lane / L;
        if (ob >= 0 && t >= olo && t < ohi && n < a.N) {
            if (AGENT)
                store_out_agent(a.y, (size_t)n, outv, a.ydt);
            else
                store_out(a.y, (size_t)n, outv, a.ydt);
        }
    };

    auto load = [&](int g, u32x4 (&q)[U], uint32_t (&sc)[U]) {
        int n = g * R + lr;
        n = n < a.N ? n : a.N - 1;
        const u32x4* cp = a.codes + (size_t)n * a.C + lk;
        const uint32_t* sp = swords + (size_t)n * Gw + sbase;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            q[u] = nt_load(cp + coff[u]);
            sc[u] = gload(sp + soff[u]);
        }
    };
    auto finish = [&](int g, const u32x4 (&q)[U], const uint32_t (&sc)[U]) {
        float acc = 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc = fmaf(scale_from_word(sc[u], ssel[u]), chunk_dot16(q[u], xr[u], k), acc);
        acc *= xv;
        if (BATCH) {
            acc = row16_sum(acc);
            const int row0 = g * R;
            const int blk = row0 & ~63;
            const int ti = (row0 - blk) / R;  // row group within the block
            if (blk != ob) {
                flush();
                ob = blk;
                olo = ti;
            }
            if (L == 16) {
                if ((lane & 15) == ti) outv = acc;
            } else if (L == 32) {
                acc += dpp_row_bcast<0x142, 0xA>(acc);  // rows 1, 3 += lanes 15, 47
                const float s0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 31));
                const float s1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 63));
                if (lane == ti) outv = s0;
                if (lane == 32 + ti) outv = s1;
            } else {
                acc += dpp_row_bcast<0x142, 0xA>(acc);  // rows 1, 3 += lanes 15, 47
                acc += dpp_row_bcast<0x143, 0xC>(acc);  // rows 2, 3 += lane 31
                const float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 63));
                if (lane == ti) outv = s;
            }
            ohi = ti + 1;
        } else {
            acc = group_sum<L>(acc);
            const int n = g * R + lr;
            if (lk == 0 && n < a.N) {
                if (AGENT)
                    store_out_agent(a.y, (size_t)n, acc, a.ydt);
                else
                    store_out(a.y, (size_t)n, acc, a.ydt);
            }
        }
    };

    // The prefetch is never skipped: on the last row group it re-reads the
    // current one (lines just fetched, so a cache hit) instead of branching.
    // A load issued under a branch that rejoins would leave the wait-count
    // pass the smaller of the two paths' counts, and the wait before decoding
    // the current row group would then also wait for the prefetched one.
    auto next = [&](int g, int d) { return g + d < rg1 ? g + d : g; };
    int rg = rg0;
    if (STAGES == 2) {
        u32x4 qa[U], qb[U];
        uint32_t sa[U], sb[U];
        load(rg, qa, sa);
        if (wave_any_inexact(x_slice_to_f16<U>(xr, xv))) {
            xs.template fallback<L>(a, rg0, rg1, step, lane);
            return;
        }
        while (true) {
            load(next(rg, step), qb, sb);
            finish(rg, qa, sa);
            rg += step;
            if (rg >= rg1) break;
            load(next(rg, step), qa, sa);
            finish(rg, qb, sb);
            rg += step;
            if (rg >= rg1) break;
        }
        if (BATCH) flush();
    } else {
        // three stages: two row groups in flight while one is decoded
        u32x4 qa[U], qb[U], qc[U];
        uint32_t sa[U], sb[U], sc[U];
        load(rg, qa, sa);
        load(next(rg, step), qb, sb);
        if (wave_any_inexact(x_slice_to_f16<U>(xr, xv))) {
            xs.template fallback<L>(a, rg0, rg1, step, lane);
            return;
        }
        while (true) {
            load(next(rg, 2 * step), qc, sc);
            finish(rg, qa, sa);
            rg += step;
            if (rg >= rg1) break;
            load(next(rg, 2 * step), qa, sa);
            finish(rg, qb, sb);
            rg += step;
            if (rg >= rg1) break;
            load(next(rg, 2 * step), qb, sb);
            finish(rg, qc, sc);
            rg += step;
            if (rg >= rg1) break;
        }
        if (BATCH) flush();
    }
}

// Any K, and the exact fallback of gemv_rows: codes decoded to bf16
// 16 (c - 8), activations used as bf16 and re-read (from cache) for every
// row, scale / 16 per chunk.  Exact products for every input, inf and NaN
// included.
template <int L>
__device__ __forceinline__ void gemv_rows_generic(const GemvArgs& a, int rg0, int rg1, int step,
                                                  int lane) {
    constexpr int R = 64 / L;
    // lane-derived offsets are formed here, not hoisted to the kernel's
    // entry, where they would stay live across the fast loops that share a
    // kernel with this one (and spill there)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lk = ln % L;
    const int lr = ln / L;
    for (int rg = rg0; rg < rg1; rg += step) {
        const int n = rg * R + lr;
        float acc = 0.f;
        if (n < a.N) {
            for (int c = lk; c < a.C; c += L) {
                const u32x4 q = nt_load(a.codes + (size_t)n * a.C + c);
                const float s =
                    bf16_to_f32(gload(a.scales + (size_t)n * a.G + (c >> a.gshift))) * 0.0625f;
                uint32_t xr[16];
                const u32x4* p = reinterpret_cast<const u32x4*>(a.x + 16 * c);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const u32x4 v = gload(p + i);
                    xr[4 * i + 0] = v[0];
                    xr[4 * i + 1] = v[1];
                    xr[4 * i + 2] = v[2];
                    xr[4 * i + 3] = v[3];
                }
                acc = fmaf(s, chunk_dot_x16(q, xr), acc);
            }
        }
        acc = group_sum<L>(acc);
        if (lk == 0 && n < a.N) store_out(a.y, (size_t)n, acc, a.ydt);
    }
}

inline GemvArgs make_gemv_args(const void* packed, int N, int K, int group, const uint16_t* x,
                               void* y, int ydt) {
    GemvArgs a;
    a.codes = static_cast<const u32x4*>(packed);
    a.scales = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(packed) +
                                                 scale_offset(N, K));
    a.x = reinterpret_cast<const uint32_t*>(x);
    a.y = y;
    a.N = N;
    a.C = K / 32;
    a.G = K / group;
    a.gshift = ilog2(group / 32);
    a.ydt = ydt;
    return a;
}

}  // namespace w4
