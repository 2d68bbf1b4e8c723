// w4_gemv.hip -- batch-1 W4A16 GEMV (M = 1) for gfx950.
//
// [P1] "Gemma 4 E2B on a 4 GB GPU with plain PyTorch, faster than llama.cpp",
// paragraph on the w4gemv.py kernel: one activation vector times a weight
// matrix read straight from its packed 4-bit words, unpacked in registers and
// multiplied, never writing a 16-bit copy; a fixed tiling per weight shape.
//
// Work split: a row of K codes is 16-byte chunks of 32 codes (one chunk = one
// dwordx4 load = one K-group of 32).  L lanes share a row; lane l of the row
// owns chunks l, l + L, ..., so for each u the L lanes read L consecutive
// chunks (L*16 contiguous bytes) and a wave reads 64/L rows at once.  A lane's
// chunks are the same for every row, so its slice of x (16 bf16 pairs per
// chunk) and the chunk's offset term stay in registers for the whole kernel.
// Rows are walked grid-stride; the next row group's codes and scales are
// loaded before the current one is reduced (two register stages).  Lane
// partials are combined in a fixed order (DPP moves within 16-lane rows), so
// results are bitwise deterministic.  Weight loads are non-temporal: each byte is read once.
#include <climits>
#include <cstdio>
#include <cstdlib>

#include "w4_dispatch.h"

namespace w4 {

struct GemvArgs {
    const u32x4* codes;      // N x C chunks (device words)
    const uint16_t* scales;  // N x G bf16
    const uint32_t* x;       // K/2 bf16 pairs
    void* y;
    int N, C, G, gshift, ydt;
};

// Loads this lane's activation slice: 16 bf16 pairs per owned chunk, and the
// chunk's offset term -136 * sum(x) (zero slices for chunks past the row).
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

// FULLC: every lane owns exactly U chunks (L * U == C).  Otherwise lanes past
// the row end read a clamped, valid chunk and multiply it by a zero
// activation slice.  Rows past N are clamped to row N - 1 and not stored, so
// the steady-state loop has no divergent branches.
template <int L, int U, bool FULLC>
__global__ __launch_bounds__(256) void gemv_xreg_kernel(GemvArgs a) {
    constexpr int R = 64 / L;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    const int lk = lane % L;
    const int lr = lane / L;
    const DecodeConsts k = decode_consts();

    uint32_t xr[U][16];
    float xb[U];
    load_x_slice<L, U>(a.x, a.C, lk, xr, xb);

    // per-u chunk and scale offsets relative to chunk lk of the row
    int coff[U], soff[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int c = lk + L * u;
        if (!FULLC && c >= a.C) c = a.C - 1;
        coff[u] = c - lk;
        soff[u] = (c >> a.gshift) - (lk >> a.gshift);
    }

    const int NG = (a.N + R - 1) / R;
    const int stride = gridDim.x * nw;
    int rg = blockIdx.x * nw + wave;
    if (rg >= NG) return;

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
            acc = fmaf(bf16_to_f32(sc[u]), chunk_dot(q[u], xr[u], xb[u], k), acc);
        acc = group_sum<L>(acc);
        const int n = g * R + lr;
        if (lk == 0 && n < a.N) store_out(a.y, (size_t)n, acc, a.ydt);
    };

    // two register stages, alternating: the next row group is in flight while
    // the current one is decoded
    u32x4 qa[U], qb[U];
    uint32_t sa[U], sb[U];
    load(rg, qa, sa);
    while (true) {
        if (rg + stride < NG) load(rg + stride, qb, sb);
        finish(rg, qa, sa);
        rg += stride;
        if (rg >= NG) break;
        if (rg + stride < NG) load(rg + stride, qa, sa);
        finish(rg, qb, sb);
        rg += stride;
        if (rg >= NG) break;
    }
}

// Any K: the activation chunk is re-read (from cache) for every row.
template <int L>
__global__ __launch_bounds__(256) void gemv_generic_kernel(GemvArgs a) {
    constexpr int R = 64 / L;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    const int lk = lane % L;
    const int lr = lane / L;
    const DecodeConsts k = decode_consts();
    const int NG = (a.N + R - 1) / R;
    for (int rg = blockIdx.x * nw + wave; rg < NG; rg += gridDim.x * nw) {
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
                acc = fmaf(s, chunk_dot(q, xr, -chunk_bias(xr), k), acc);
            }
        }
        acc = group_sum<L>(acc);
        if (lk == 0 && n < a.N) store_out(a.y, (size_t)n, acc, a.ydt);
    }
}

template <int L, int U>
static void launch_xreg_LU(bool full, dim3 g, dim3 b, hipStream_t s, const GemvArgs& a) {
    if (full)
        gemv_xreg_kernel<L, U, true><<<g, b, 0, s>>>(a);
    else
        gemv_xreg_kernel<L, U, false><<<g, b, 0, s>>>(a);
}

template <int L>
static void launch_xreg_L(int U, dim3 g, dim3 b, hipStream_t s, const GemvArgs& a) {
    const bool full = L * U == a.C;
    switch (U) {
        case 1: launch_xreg_LU<L, 1>(full, g, b, s, a); break;
        case 2: launch_xreg_LU<L, 2>(full, g, b, s, a); break;
        case 3: launch_xreg_LU<L, 3>(full, g, b, s, a); break;
        case 4: launch_xreg_LU<L, 4>(full, g, b, s, a); break;
        case 5: launch_xreg_LU<L, 5>(full, g, b, s, a); break;
        case 6: launch_xreg_LU<L, 6>(full, g, b, s, a); break;
        case 7: launch_xreg_LU<L, 7>(full, g, b, s, a); break;
        default: launch_xreg_LU<L, 8>(full, g, b, s, a); break;
    }
}

static bool env_tile(GemvTile& t) {
    const char* e = getenv("W4_GEMV_TILE");
    if (!e || !*e) return false;
    int L, U, W;
    if (sscanf(e, "%d,%d,%d", &L, &U, &W) != 3) return false;
    if ((L != 8 && L != 16 && L != 32 && L != 64) || U < 1 || U > kMaxU ||
        W < 1 || W > 4)
        return false;
    t.L = L;
    t.U = U;
    t.waves = W;
    return true;
}

static int waves_per_cu() {
    const char* e = getenv("W4_GEMV_WAVES_PER_CU");
    int v = e ? atoi(e) : 0;
    return (v >= 1 && v <= 32) ? v : 8;
}

GemvTile pick_gemv_tile(int N, int K, int group) {
    (void)group;
    GemvTile t;
    const int C = K / 32;
    const int target = kNumCUs * waves_per_cu();
    if (!env_tile(t)) {
        // Zero-waste splits (every lane owns the same number of chunks), in
        // order of preference; when the first leaves the chip short of waves,
        // take the zero-waste split with the most row groups.
        static const int order[4] = {16, 64, 32, 8};
        int cand[4], nc = 0, best_waste = INT_MAX;
        for (int L : order) {
            const int U = (C + L - 1) / L;
            if (U > kMaxU) continue;
            const int waste = L * U - C;
            if (waste < best_waste) {
                best_waste = waste;
                nc = 0;
            }
            if (waste == best_waste) cand[nc++] = L;
        }
        if (nc == 0) {
            t.L = 64;
            t.U = 0;
            t.generic = true;
        } else {
            int L = cand[0];
            const int ng0 = (N + 64 / L - 1) / (64 / L);
            if (ng0 < target) {
                for (int i = 1; i < nc; ++i)
                    if (cand[i] > L) L = cand[i];
            }
            t.L = L;
            t.U = (C + L - 1) / L;
        }
        t.waves = 4;
    } else if (t.L * t.U < C) {
        t.generic = true;
    }
    const int R = 64 / t.L;
    const int NG = (N + R - 1) / R;
    const int waves = NG < target ? NG : target;
    t.grid = (waves + t.waves - 1) / t.waves;
    if (t.grid < 1) t.grid = 1;
    return t;
}

int launch_gemv(const GemvTile& t, const void* packed, int N, int K, int group,
                const uint16_t* x, void* y, int ydt, hipStream_t s) {
    GemvArgs a;
    a.codes = static_cast<const u32x4*>(packed);
    a.scales = reinterpret_cast<const uint16_t*>(
        static_cast<const uint8_t*>(packed) + scale_offset(N, K));
    a.x = reinterpret_cast<const uint32_t*>(x);
    a.y = y;
    a.N = N;
    a.C = K / 32;
    a.G = K / group;
    a.gshift = ilog2(group / 32);
    a.ydt = ydt;
    const dim3 g(t.grid), b(64 * t.waves);
    if (t.generic) {
        switch (t.L) {
            case 8: gemv_generic_kernel<8><<<g, b, 0, s>>>(a); break;
            case 16: gemv_generic_kernel<16><<<g, b, 0, s>>>(a); break;
            case 32: gemv_generic_kernel<32><<<g, b, 0, s>>>(a); break;
            default: gemv_generic_kernel<64><<<g, b, 0, s>>>(a); break;
        }
    } else {
        switch (t.L) {
            case 8: launch_xreg_L<8>(t.U, g, b, s, a); break;
            case 16: launch_xreg_L<16>(t.U, g, b, s, a); break;
            case 32: launch_xreg_L<32>(t.U, g, b, s, a); break;
            default: launch_xreg_L<64>(t.U, g, b, s, a); break;
        }
    }
    return hip_fail(hipGetLastError(), "gemv launch");
}

}  // namespace w4
