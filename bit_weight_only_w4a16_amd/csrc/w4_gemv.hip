// w4_gemv.hip -- batch-1 W4A16 GEMV (M = 1) for gfx950.
//
// [P1] "Gemma 4 E2B on a 4 GB GPU with plain PyTorch, faster than llama.cpp",
// paragraph on the w4gemv.py kernel: one activation vector times a weight
// matrix read straight from its packed 4-bit words, unpacked in registers and
// multiplied, never writing a 16-bit copy; a fixed tiling per weight shape.
//
// The work split and inner loop are in w4_gemv_core.h; this file holds the
// stand-alone kernels (row groups walked grid-stride over the whole grid) and
// the per-shape tile table.

#include <climits>
#include <cstdio>
#include <cstdlib>

#include "w4_config.h"
#include "w4_gemv_core.h"

namespace w4 {

#include "w4_tiles.h"

// The built-in table's tile for a shape, if any.
static bool builtin_tile(int N, int K, int group, GemvTile& t) {
    for (int i = 0; i < kBuiltinTileCount; ++i) {
        const TileEntry& e = kBuiltinTiles[i];
        if (e.N == N && e.K == K && e.group == group) {
            t = e.t;
            return true;
        }
    }
    return false;
}

template <int L, int U, bool FULLC, int STAGES>
__global__ __launch_bounds__(256) void gemv_xreg_kernel(GemvArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    const DecodeConsts k = decode_consts();
    const int NG = (a.N + 64 / L - 1) / (64 / L);
    gemv_rows<L, U, FULLC, STAGES>(a, blockIdx.x * nw + wave, NG, gridDim.x * nw, lane, k);
}

// Large matrices (e.g. a 262144-row output layer): every wave streams one
// contiguous range of row groups with the next row group in flight and the
// outputs written in 64-row blocks, as one op of the decode-step stream
// kernel does; 16 waves per CU (<= 128 VGPRs).
template <int L, int U, int STAGES>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
void gemv_contig_kernel(GemvArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    const DecodeConsts k = decode_consts();
    const int NG = (a.N + 64 / L - 1) / (64 / L);
    const long long W = (long long)gridDim.x * nw, w = (long long)blockIdx.x * nw + wave;
    const int rg0 = (int)(w * NG / W), rg1 = (int)((w + 1) * NG / W);
    gemv_rows<L, U, true, STAGES, true>(a, rg0, rg1, 1, lane, k);
}

template <int L>
__global__ __launch_bounds__(256) void gemv_generic_kernel(GemvArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    const int NG = (a.N + 64 / L - 1) / (64 / L);
    gemv_rows_generic<L>(a, blockIdx.x * nw + wave, NG, gridDim.x * nw, lane);
}

// Row groups from which a full-width tiling of at most 3 chunks per lane
// streams contiguous ranges: 16 per wave of 16 waves per CU.
constexpr int kContigWaves = kNumCUs * 16;
constexpr int kContigRowGroups = 16 * kContigWaves;

template <int L, int U>
static void contig_launch(int stages, dim3 g, hipStream_t s, const GemvArgs& a) {
    if constexpr (U <= 3) {
        if (stages == 3)
            gemv_contig_kernel<L, U, 3><<<g, dim3(256), 0, s>>>(a);
        else
            gemv_contig_kernel<L, U, 2><<<g, dim3(256), 0, s>>>(a);
    }
}

template <int L, int U, bool FULLC>
static void xreg_launch(int stages, dim3 g, dim3 b, hipStream_t s, const GemvArgs& a) {
    if constexpr (U <= 4) {
        if (stages == 3) {
            gemv_xreg_kernel<L, U, FULLC, 3><<<g, b, 0, s>>>(a);
            return;
        }
    }
    gemv_xreg_kernel<L, U, FULLC, 2><<<g, b, 0, s>>>(a);
}

template <int L, int U>
static void launch_xreg_LU(bool full, bool contig, int stages, dim3 g, dim3 b, hipStream_t s,
                           const GemvArgs& a) {
    if (contig) {
        contig_launch<L, U>(stages, g, s, a);
        return;
    }
    if (full)
        xreg_launch<L, U, true>(stages, g, b, s, a);
    else
        xreg_launch<L, U, false>(stages, g, b, s, a);
}

template <int L>
static void launch_xreg_L(int U, bool contig, int stages, dim3 g, dim3 b, hipStream_t s,
                          const GemvArgs& a) {
    const bool full = L * U == a.C;
    switch (U) {
        case 1: launch_xreg_LU<L, 1>(full, contig, stages, g, b, s, a); break;
        case 2: launch_xreg_LU<L, 2>(full, contig, stages, g, b, s, a); break;
        case 3: launch_xreg_LU<L, 3>(full, contig, stages, g, b, s, a); break;
        case 4: launch_xreg_LU<L, 4>(full, contig, stages, g, b, s, a); break;
        case 5: launch_xreg_LU<L, 5>(full, contig, stages, g, b, s, a); break;
        case 6: launch_xreg_LU<L, 6>(full, contig, stages, g, b, s, a); break;
        case 7: launch_xreg_LU<L, 7>(full, contig, stages, g, b, s, a); break;
        default: launch_xreg_LU<L, 8>(full, contig, stages, g, b, s, a); break;
    }
}

// The heuristic tile: the zero-waste lane split (every lane owns the same
// number of chunks) in order of preference 16, 64, 32, 8 lanes per row; when
// the first leaves the chip short of waves, the zero-waste split with the
// most row groups.  A K with no tiling, or an odd number of groups per row
// (the tiled loop reads scales in dword pairs), takes the generic loop.
// Large matrices whose tile covers a row exactly with at most 3 chunks per
// lane and 16 or more lanes per row (the row sums of the contiguous kernel's
// output gathering) stream contiguous row ranges (contig).
static GemvTile heuristic_tile(int N, int K, int group, bool allow_contig) {
    GemvTile t;
    const int C = K / 32;
    const int target = kNumCUs * 8;
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
    if (nc == 0 || ((K / group) & 1)) {
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
    const int NG = (N + 64 / t.L - 1) / (64 / t.L);
    t.contig = allow_contig && !t.generic && t.L >= 16 && t.L * t.U == C && t.U <= 3 &&
               NG >= kContigRowGroups;
    t.grid = 0;
    return t;
}

// grid 0: the contiguous kernel runs 16 waves per CU; the grid-stride kernels
// one wave per row group, at most 8 per CU
static void auto_grid(GemvTile& t, int N) {
    if (t.grid > 0) return;
    if (t.contig) {
        t.grid = kContigWaves / 4;
        return;
    }
    const int NG = (N + 64 / t.L - 1) / (64 / t.L);
    const int target = kNumCUs * 8;
    const int waves = NG < target ? NG : target;
    t.grid = (waves + t.waves - 1) / t.waves;
    if (t.grid < 1) t.grid = 1;
}

GemvTile pick_gemv_tile(int N, int K, int group, const char** source) {
    const auto cfg = config();
    GemvTile t;
    const char* src = "heuristic";
    if (cfg->force & kForceGemvGeneric) {
        t.L = 64;
        t.U = 0;
        t.generic = true;
        t.waves = 4;
        t.grid = 0;
        src = "forced gemv_generic";
    } else if (cfg->force & (kForceGemvTiled | kForceGemvContig)) {
        t = heuristic_tile(N, K, group, (cfg->force & kForceGemvContig) != 0);
        src = (cfg->force & kForceGemvContig) ? "forced gemv_contig" : "forced gemv_tiled";
    } else if (table_tile(*cfg, N, K, group, t)) {
        src = "table";
    } else if (builtin_tile(N, K, group, t)) {
        src = "built-in table";
    } else {
        t = heuristic_tile(N, K, group, true);
    }
    auto_grid(t, N);
    if (source) *source = src;
    return t;
}

int launch_gemv(const GemvTile& t, const void* packed, int N, int K, int group,
                const uint16_t* x, void* y, int ydt, hipStream_t s) {
    const GemvArgs a = make_gemv_args(packed, N, K, group, x, y, ydt);
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
            case 8: launch_xreg_L<8>(t.U, t.contig, t.stages, g, b, s, a); break;
            case 16: launch_xreg_L<16>(t.U, t.contig, t.stages, g, b, s, a); break;
            case 32: launch_xreg_L<32>(t.U, t.contig, t.stages, g, b, s, a); break;
            default: launch_xreg_L<64>(t.U, t.contig, t.stages, g, b, s, a); break;
        }
    }
    return hip_fail(hipGetLastError(), "gemv launch");
}

}  // namespace w4
