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
// chunks are the same for every row, so its activation slice (16 bf16 pairs
// per chunk) and the chunks' offset terms stay in registers.
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

// Loads this lane's activation slice and the negated offset terms
// -136 * sum(x) (zero slices for chunks past the row end).
template <int L, int U>
__device__ __forceinline__ void load_x_slice(const uint32_t* x, int C, int lk,
                                             uint32_t (&xr)[U][16], float (&xb)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = lk + L * u;
        if (c < C) {
            const u32x4* p = reinterpret_cast<const u32x4*>(x + 16 * c);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x4 v = p[i];
                xr[u][4 * i + 0] = v[0];
                xr[u][4 * i + 1] = v[1];
                xr[u][4 * i + 2] = v[2];
                xr[u][4 * i + 3] = v[3];
            }
            xb[u] = -chunk_bias(xr[u]);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) xr[u][i] = 0u;
            xb[u] = 0.f;
        }
    }
}

// Row groups rg0, rg0 + step, ... (< rg1) of one matrix for one wave.
// FULLC: L * U == C.  Otherwise lanes past the row end read a clamped, valid
// chunk and multiply it by a zero activation slice.  Rows past N are clamped
// to row N - 1 and not stored, so the loop has no divergent branches.
// STAGES register sets rotate: STAGES - 1 row groups are in flight while the
// current one is decoded.  Lane partials are summed in a fixed order, so the
// result is bitwise deterministic.
template <int L, int U, bool FULLC, int STAGES = 2>
__device__ __forceinline__ void gemv_rows(const GemvArgs& a, int rg0, int rg1, int step,
                                          int lane, const DecodeConsts& k) {
    static_assert(STAGES == 2 || STAGES == 3, "register stages");
    constexpr int R = 64 / L;
    const int lk = lane % L;
    const int lr = lane / L;
    if (rg0 >= rg1) return;

    uint32_t xr[U][16];
    float xb[U];
    load_x_slice<L, U>(a.x, a.C, lk, xr, xb);

    int coff[U], soff[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int c = lk + L * u;
        if (!FULLC && c >= a.C) c = a.C - 1;
        coff[u] = c - lk;
        soff[u] = (c >> a.gshift) - (lk >> a.gshift);
    }

    auto load = [&](int g, u32x4 (&q)[U], uint32_t (&sc)[U]) {
        int n = g * R + lr;
        n = n < a.N ? n : a.N - 1;
        const u32x4* cp = a.codes + (size_t)n * a.C + lk;
        const uint16_t* sp = a.scales + (size_t)n * a.G + (lk >> a.gshift);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            q[u] = nt_load(cp + coff[u]);
            sc[u] = sp[soff[u]];
        }
    };
    auto finish = [&](int g, const u32x4 (&q)[U], const uint32_t (&sc)[U]) {
        float acc = 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc = fmaf(bf16_to_f32(sc[u]), chunk_dot(q[u], xr[u], k) + xb[u], acc);
        acc = group_sum<L>(acc);
        const int n = g * R + lr;
        if (lk == 0 && n < a.N) store_out(a.y, (size_t)n, acc, a.ydt);
    };

    int rg = rg0;
    if (STAGES == 2) {
        u32x4 qa[U], qb[U];
        uint32_t sa[U], sb[U];
        load(rg, qa, sa);
        while (true) {
            if (rg + step < rg1) load(rg + step, qb, sb);
            finish(rg, qa, sa);
            rg += step;
            if (rg >= rg1) break;
            if (rg + step < rg1) load(rg + step, qa, sa);
            finish(rg, qb, sb);
            rg += step;
            if (rg >= rg1) break;
        }
    } else {
        // three stages: two row groups in flight while one is decoded
        u32x4 qa[U], qb[U], qc[U];
        uint32_t sa[U], sb[U], sc[U];
        load(rg, qa, sa);
        if (rg + step < rg1) load(rg + step, qb, sb);
        while (true) {
            if (rg + 2 * step < rg1) load(rg + 2 * step, qc, sc);
            finish(rg, qa, sa);
            rg += step;
            if (rg >= rg1) break;
            if (rg + 2 * step < rg1) load(rg + 2 * step, qa, sa);
            finish(rg, qb, sb);
            rg += step;
            if (rg >= rg1) break;
            if (rg + 2 * step < rg1) load(rg + 2 * step, qb, sb);
            finish(rg, qc, sc);
            rg += step;
            if (rg >= rg1) break;
        }
    }
}

// Any K: the activation chunk is re-read (from cache) for every row.
template <int L>
__device__ __forceinline__ void gemv_rows_generic(const GemvArgs& a, int rg0, int rg1, int step,
                                                  int lane, const DecodeConsts& k) {
    constexpr int R = 64 / L;
    const int lk = lane % L;
    const int lr = lane / L;
    for (int rg = rg0; rg < rg1; rg += step) {
        const int n = rg * R + lr;
        float acc = 0.f;
        if (n < a.N) {
            for (int c = lk; c < a.C; c += L) {
                const u32x4 q = nt_load(a.codes + (size_t)n * a.C + c);
                const float s = bf16_to_f32(a.scales[(size_t)n * a.G + (c >> a.gshift)]);
                uint32_t xr[16];
                const u32x4* p = reinterpret_cast<const u32x4*>(a.x + 16 * c);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const u32x4 v = p[i];
                    xr[4 * i + 0] = v[0];
                    xr[4 * i + 1] = v[1];
                    xr[4 * i + 2] = v[2];
                    xr[4 * i + 3] = v[3];
                }
                acc = fmaf(s, chunk_dot(q, xr, k) - chunk_bias(xr), acc);
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
