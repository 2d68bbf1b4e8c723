// w4_smallm.hip -- W4A16 product for 2 <= M <= 16 activation rows.
//
// [P2] "fastgemma -- Gemma 4 E2B, CPU-only, AMX INT8 / AVX-512 VNNI", section
// "Why AMX for GEMM but not for attention": a weight GEMM reuses each weight
// byte across all M rows.  Each packed chunk is loaded and decoded once to
// the exact bf16 operand pairs 16 (c - 8) (w4_common.h), then multiplied by
// every activation row; each chunk's sum is scaled by s / 16.
//
// Work split as in the batch-1 GEMV: L lanes share a weight row (lane l owns
// chunks l, l + L, ...), a wave covers 64/L rows per step.  The activation
// rows are staged once per workgroup in LDS when they fit; otherwise
// (generic kernel) they are read through the cache.  At this size the kernel
// is bound by vector ALU work (one dot2 per two codes per row).
#include <cstdio>
#include <cstdlib>

#include "w4_config.h"
#include "w4_dispatch.h"
#include "w4_fwht.h"

namespace w4 {

constexpr int kSmL = 16;                 // lanes per weight row
constexpr size_t kSmLdsMax = 64 * 1024;  // LDS budget of one workgroup

struct SmallMArgs {
    const u32x4* codes;
    const uint16_t* scales;
    const uint16_t* X;
    void* Y;
    int N, C, G, gshift, M, ldx, ldy, ydt, K;
};

template <int MT, bool XLDS>
__global__ __launch_bounds__(256) void smallm_kernel(SmallMArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int L = kSmL, R = 64 / kSmL;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    const int lk = lane % L;
    const int lr = lane / L;

    uint32_t* xs = reinterpret_cast<uint32_t*>(smem);                   // [M][K/2]
    if (XLDS) {
        const int vec_per_row = a.K / 8;  // u32x4 per row
        for (int i = threadIdx.x; i < a.M * vec_per_row; i += blockDim.x) {
            const int m = i / vec_per_row, v = i % vec_per_row;
            const u32x4 val = reinterpret_cast<const u32x4*>(a.X + (size_t)m * a.ldx)[v];
            reinterpret_cast<u32x4*>(xs)[i] = val;
        }
        __syncthreads();
    }

    const int NG = (a.N + R - 1) / R;
    for (int rg = blockIdx.x * nw + wave; rg < NG; rg += gridDim.x * nw) {
        const int n = rg * R + lr;
        float acc[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = 0.f;
        if (n < a.N) {
            for (int c = lk; c < a.C; c += L) {
                const u32x4 q = nt_load(a.codes + (size_t)n * a.C + c);
                const float s =
                    bf16_to_f32(a.scales[(size_t)n * a.G + (c >> a.gshift)]) * 0.0625f;
                uint32_t d[16];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const u32x4 b = decode_x16(q[w]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) d[4 * w + j] = b[j];
                }
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    if (m < a.M) {
                        uint32_t xr[16];
                        if (XLDS) {
                            const u32x4* p = reinterpret_cast<const u32x4*>(
                                xs + (size_t)m * (a.K / 2) + c * 16);
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const u32x4 v = p[i];
                                xr[4 * i + 0] = v[0];
                                xr[4 * i + 1] = v[1];
                                xr[4 * i + 2] = v[2];
                                xr[4 * i + 3] = v[3];
                            }
                        } else {
                            const u32x4* p = reinterpret_cast<const u32x4*>(
                                a.X + (size_t)m * a.ldx + (size_t)c * 32);
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const u32x4 v = p[i];
                                xr[4 * i + 0] = v[0];
                                xr[4 * i + 1] = v[1];
                                xr[4 * i + 2] = v[2];
                                xr[4 * i + 3] = v[3];
                            }
                        }
                        float d0 = 0.f, d1 = 0.f;
#pragma unroll
                        for (int i = 0; i < 16; i += 2) {
                            d0 = dot2(d[i], xr[i], d0);
                            d1 = dot2(d[i + 1], xr[i + 1], d1);
                        }
                        acc[m] = fmaf(s, d0 + d1, acc[m]);
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
#pragma unroll
            for (int off = L / 2; off > 0; off >>= 1) acc[m] += __shfl_xor(acc[m], off, 64);
        }
        if (lk == 0 && n < a.N) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (m < a.M) store_out(a.Y, (size_t)m * a.ldy + n, acc[m], a.ydt);
        }
    }
}

// Fast path: every lane owns exactly U chunks (C == L * U) and X fits LDS.
// The row group's codes and scales for all U chunks are loaded at once, with
// the next row group in flight (two register stages), so a wave pays one
// memory latency per row group, not one per chunk.  Each chunk is decoded
// once into 16 operand pairs and multiplied by the M activation rows read
// from LDS (lanes of the same chunk read the same LDS words).  The M sums of
// a row are reduced with DPP moves; lane m of the row then stores output m.
template <int MT, int L, int U>
__global__ __launch_bounds__(256) void smallm_fast_kernel(SmallMArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int R = 64 / L;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    const int lk = lane % L;
    const int lr = lane / L;

    // X in LDS, one 64-byte chunk per (row m, chunk c); quarter i of chunk c
    // is stored at quarter (i + c/2) mod 4, so the 16-byte reads of eight
    // consecutive chunks (one per lane of an 8-lane group) hit all 32 banks.
    uint32_t* xs = reinterpret_cast<uint32_t*>(smem);                   // [M][C][16]
    {
        const int vec_per_row = a.K / 8;
        for (int i = threadIdx.x; i < a.M * vec_per_row; i += blockDim.x) {
            const int m = i / vec_per_row, v = i % vec_per_row;
            const int c = v >> 2, q = v & 3;
            reinterpret_cast<u32x4*>(xs)[((size_t)m * a.C + c) * 4 + ((q + (c >> 1)) & 3)] =
                reinterpret_cast<const u32x4*>(a.X + (size_t)m * a.ldx)[v];
        }
        __syncthreads();
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
            q[u] = nt_load(cp + L * u);
            sc[u] = sp[(L * u) >> a.gshift];
        }
    };
    auto finish = [&](int g, const u32x4 (&q)[U], const uint32_t (&sc)[U]) {
        float acc[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = lk + L * u;
            uint32_t d[16];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const u32x4 b = decode_x16(q[u][w]);
#pragma unroll
                for (int j = 0; j < 4; ++j) d[4 * w + j] = b[j];
            }
            const float s = bf16_to_f32(sc[u]) * 0.0625f;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (m < a.M) {
                    const u32x4* p =
                        reinterpret_cast<const u32x4*>(xs) + ((size_t)m * a.C + c) * 4;
                    uint32_t xr[16];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const u32x4 v = p[(i + (c >> 1)) & 3];
                        xr[4 * i + 0] = v[0];
                        xr[4 * i + 1] = v[1];
                        xr[4 * i + 2] = v[2];
                        xr[4 * i + 3] = v[3];
                    }
                    float d0 = 0.f, d1 = 0.f;
#pragma unroll
                    for (int i = 0; i < 16; i += 2) {
                        d0 = dot2(d[i], xr[i], d0);
                        d1 = dot2(d[i + 1], xr[i + 1], d1);
                    }
                    acc[m] = fmaf(s, d0 + d1, acc[m]);
                }
            }
        }
        float mine = 0.f;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const float t = group_sum<L>(acc[m]);
            if (lk == m) mine = t;
        }
        const int n = g * R + lr;
        if (lk < a.M && n < a.N) store_out(a.Y, (size_t)lk * a.ldy + n, mine, a.ydt);
    };

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


// ------------------------------------------------ matrix-core small M ---
//
// Groups 32, 256 and 512, M <= 16: one 16-row MFMA tile holds every
// activation row (rows past M repeat row M - 1 and are never stored), so the
// matrix cores do the per-row work the vector-ALU kernel spends its time on.
// v_mfma_f32_16x16x32_bf16 (lane l holds A[l%16][8(l/16) + j],
// B[8(l/16) + j][l%16], D[4(l/16) + r][l%16]); codes decoded to the exact
// bf16 values 16 (c - 8), each group's product scaled by s / 16, as in the
// prefill kernels.
//
// A workgroup owns 16 * RG weight rows and splits K into KS slices: wave
// (row group rg, slice ks) multiplies 16 rows by its 128 * NB slice of K.
// Each wave loads all of its codes before anything else, so a workgroup's
// whole weight stream is in flight at once.  Groups of 256 and 512: 16 bytes
// per lane per 128-K block, lane group l/16 taking words 4(l/16) .. 4(l/16) +
// 3 of its row's block and using word t in MFMA step t (the activations read
// with the same K permutation).  Group 32 (G32): MFMA step t of a block must
// cover exactly group t, so lane group l/16 needs word 4t + l/16: the same
// 16-byte loads, then a 4 x 4 transpose of the words across the four lane
// groups (two exchange steps, lanes 16 and 32 apart); every step closes its
// group.  The activation rows are staged once per workgroup in LDS, 16-byte
// chunk q of row m at position q ^ (m & 15) (fragment reads conflict-free).
// The slices' results are added through LDS in slice order 0, 1, ..., so
// the output is deterministic.
struct SmqArgs {
    const uint8_t* codes;    // N x K/2 bytes (device words)
    const uint16_t* scales;  // N x G bf16
    const uint16_t* X;       // M x K bf16, row stride ldx
    void* Y;
    int N, K, G, group, M, ldx, ldy, ydt;
    int RG, KS;              // row groups and K slices per workgroup
    int had;                 // 512: transform the staged rows (blockwise FWHT) first (HAD)
    float hscale;            // 512^-1/2
};
constexpr int kSmqXPer = 8;                      // activation chunks per thread and round
constexpr size_t kSmqLds = 160 * 1024;           // activation rows + slice sums, at most

template <int NB, bool HAD, bool G32>
__global__ __launch_bounds__(1024) void smallm_mfma_kernel(SmqArgs a) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    extern __shared__ __align__(16) uint8_t smem[];
    const int nthr = blockDim.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lk = lane >> 4;
    const int rg = wave % a.RG, ks = wave / a.RG;
    const int n0 = blockIdx.x * 16 * a.RG;
    const int n = min(n0 + 16 * rg + li, a.N - 1);
    constexpr int KR = 128 * NB;                 // K per wave
    const int k0 = ks * KR;
    const int CPR = a.K / 8;                     // 16-byte chunks per activation row
    const int GW = KR / a.group;                 // groups per wave (1 or 2)

    // codes and scales of this lane's row and slice: issued first
    u32x4 q[NB];
    uint32_t sc[G32 ? 2 * NB : 2];
    if (G32) {
        // words 4lk .. 4lk + 3 of each block (transposed below), and the
        // scales of groups 4u .. 4u + 3 as one 8-byte load per block (row
        // and slice offsets are multiples of 4 groups: K % 128 == 0)
        const uint8_t* crow = a.codes + (size_t)n * (a.K / 2) + k0 / 2 + 16 * lk;
#pragma unroll
        for (int u = 0; u < NB; ++u) q[u] = nt_load(reinterpret_cast<const u32x4*>(crow + 64 * u));
        const u32x2* srow =
            reinterpret_cast<const u32x2*>(a.scales + (size_t)n * a.G + k0 / 32);
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const u32x2 v = gload(srow + u);
            sc[2 * u] = v[0];
            sc[2 * u + 1] = v[1];
        }
    } else {
        const uint8_t* crow = a.codes + (size_t)n * (a.K / 2) + k0 / 2 + 16 * lk;
#pragma unroll
        for (int u = 0; u < NB; ++u) q[u] = nt_load(reinterpret_cast<const u32x4*>(crow + 64 * u));
        sc[0] = gload(a.scales + (size_t)n * a.G + k0 / a.group);
        sc[1] = gload(a.scales + (size_t)n * a.G + (k0 + KR - 1) / a.group);
    }

    // activation rows -> LDS, in rounds of kSmqXPer chunks per thread (all of
    // a round's loads before its stores)
    const int total = a.M * CPR;
    auto stage_round = [&](int e0) {
        u32x4 xv[kSmqXPer];
#pragma unroll
        for (int i = 0; i < kSmqXPer; ++i) {
            const int e = e0 + tid + i * nthr;
            if (e < total) {
                const int m = e / CPR, c = e - m * CPR;
                xv[i] = gload(reinterpret_cast<const u32x4*>(a.X + (size_t)m * a.ldx) + c);
            }
        }
#pragma unroll
        for (int i = 0; i < kSmqXPer; ++i) {
            const int e = e0 + tid + i * nthr;
            if (e < total) {
                const int m = e / CPR, c = e - m * CPR;
                reinterpret_cast<u32x4*>(smem)[m * CPR + (c ^ (m & 15))] = xv[i];
            }
        }
    };
    if (total <= kSmqXPer * nthr)
        stage_round(0);
    else
        for (int e0 = 0; e0 < total; e0 += kSmqXPer * nthr) stage_round(e0);
    __syncthreads();

    // The run-time Hadamard transform of the staged rows, in place: one wave
    // per (row, 512-block), lane l holding the block's 16-byte chunk l, with
    // the transform kernel's butterflies, scale and rounding, so the rows
    // are bitwise those that kernel writes.
    if (HAD) {
        const int nbk = a.K / 512;
        const int nwv = nthr >> 6;
        for (int job = wave; job < a.M * nbk; job += nwv) {
            const int m = job / nbk, b = job - m * nbk;
            u32x4* p = reinterpret_cast<u32x4*>(smem) + m * CPR + ((b * 64 + lane) ^ (m & 15));
            const u32x4 w = *p;
            float v[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = __uint_as_float(w[i] << 16);
                v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
            }
            fwht_block<8>(v, lane, 64);
            u32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                o[i] = f32_to_bf16_rne(v[2 * i] * a.hscale) |
                       (f32_to_bf16_rne(v[2 * i + 1] * a.hscale) << 16);
            *p = o;
        }
        __syncthreads();
    }

    const int xm = min(li, a.M - 1);             // A-operand row of this lane
    const u32x4* xrow = reinterpret_cast<const u32x4*>(smem) + (size_t)xm * CPR;
    const int xsw = xm & 15;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 tot = zero, acc = zero;
    if (G32) {
        // Lane group r holds row r of the block's 4 x 4 word matrix
        // M[r][c] = word 4r + c; two exchange steps leave it column r,
        // q[u][t] = M[t][r] = word 4t + r.  Step 1 pairs lane groups r, r ^ 1
        // (lanes 16 apart) and swaps M[even r][odd c] with M[odd r][even c];
        // step 2 pairs r, r ^ 2 (lanes 32 apart) and swaps positions 2, 3 of
        // the lower pair with positions 0, 1 of the upper pair.
        const bool b0 = (lk & 1) != 0, b1 = (lk & 2) != 0;
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            u32x4 v = q[u];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t snd = b0 ? v[2 * h] : v[2 * h + 1];
                const uint32_t rcv = (uint32_t)__shfl_xor((int)snd, 16, 64);
                if (b0)
                    v[2 * h] = rcv;
                else
                    v[2 * h + 1] = rcv;
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t snd = b1 ? v[h] : v[2 + h];
                const uint32_t rcv = (uint32_t)__shfl_xor((int)snd, 32, 64);
                if (b1)
                    v[h] = rcv;
                else
                    v[2 + h] = rcv;
            }
            q[u] = v;
        }
#pragma unroll
        for (int u = 0; u < NB; ++u)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int cq = (k0 + 128 * u + 32 * t + 8 * lk) / 8;
                const u32x4 xa = xrow[cq ^ xsw];
                const u32x4 bv = decode_x16(q[u][t]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa),
                                                              __builtin_bit_cast(bf16x8, bv),
                                                              zero, 0, 0, 0);
                const uint32_t sw = sc[2 * u + (t >> 1)];
                const float s =
                    __uint_as_float((t & 1) ? (sw & 0xFFFF0000u) : (sw << 16)) * 0.0625f;
#pragma unroll
                for (int r = 0; r < 4; ++r) tot[r] = fmaf(s, acc[r], tot[r]);
            }
    }
    const int bpg = a.group / 128;               // blocks per group
#pragma unroll
    for (int u = 0; u < NB && !G32; ++u) {
        const bool first = (u % bpg) == 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int cq = (k0 + 128 * u + 32 * lk + 8 * t) / 8;
            const u32x4 xa = xrow[cq ^ xsw];
            const u32x4 bv = decode_x16(q[u][t]);
            const bool z = first && t == 0;
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa),
                                                          __builtin_bit_cast(bf16x8, bv),
                                                          z ? zero : acc, 0, 0, 0);
        }
        if ((u + 1) % bpg == 0) {
            const float s = bf16_to_f32(sc[GW > 1 && u >= bpg ? 1 : 0]) * 0.0625f;
#pragma unroll
            for (int r = 0; r < 4; ++r) tot[r] = fmaf(s, acc[r], tot[r]);
        }
    }

    // slices summed in order 0 .. KS - 1
    f32x4* red = reinterpret_cast<f32x4*>(smem + (size_t)a.M * a.K * 2);
    if (a.KS > 1) {
        red[(ks * a.RG + rg) * 64 + lane] = tot;
        __syncthreads();
        if (ks != 0) return;
        tot = red[rg * 64 + lane];
        for (int j = 1; j < a.KS; ++j) {
            const f32x4 o = red[(j * a.RG + rg) * 64 + lane];
#pragma unroll
            for (int r = 0; r < 4; ++r) tot[r] += o[r];
        }
    }
    const int nn = n0 + 16 * rg + li;
    if (nn < a.N) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * lk + r;
            if (m < a.M) store_out(a.Y, (size_t)m * a.ldy + nn, tot[r], a.ydt);
        }
    }
}

struct SmqPlan {
    bool ok;
    int NB, RG, KS, grid;
    size_t lds;
};

// The matrix-core small-M plan, when the shape allows it: groups of 32, 256
// or 512, each wave's K slice (<= 512) a whole number of 128-K blocks and of
// groups, the activation rows within the LDS budget (a CU's 160 KB).  Group
// 32 from 5 rows: below that the vector-ALU kernel measured faster (N = 12288,
// K = 1536: 5.0 against 6.2 us at 2 rows, 10.1 against 6.7 us at 8).
static SmqPlan plan_smq(int M, int N, int K, int group) {
    SmqPlan p{};
    p.ok = false;
    if (M > 16 || (group != 32 && group != 256 && group != 512) || K % 128 != 0) return p;
    if (group == 32 && M < 5) return p;
    const int units = group == 32 ? K / 128 : K / group;   // slices hold whole units
    int KS = 0;
    for (int ks = 1; ks <= 16 && ks <= units; ++ks)
        if (units % ks == 0 && K / ks <= 512) {
            KS = ks;
            break;
        }
    if (KS == 0) return p;
    int RG = 1;
    for (int r = 4; r >= 1; --r)
        if (r * KS <= 16 && (N + 16 * r - 1) / (16 * r) >= kNumCUs) {
            RG = r;
            break;
        }
    const size_t xl = (size_t)M * K * 2;
    if (xl + (size_t)KS * RG * 64 * 16 > kSmqLds) return p;
    p.ok = true;
    p.KS = KS;
    p.RG = RG;
    p.NB = K / KS / 128;
    p.grid = (N + 16 * RG - 1) / (16 * RG);
    p.lds = xl + (size_t)KS * RG * 64 * 16;
    return p;
}

bool smallm_mfma_applies(int M, int N, int K, int group) {
    return plan_smq(M, N, K, group).ok && !(config()->force & kForceSmallmValu);
}

static size_t smallm_lds(int M, int K) {
    return (size_t)M * K * 2;
}

static int smallm_grid(int N, int R = 4) {
    const int NG = (N + R - 1) / R;
    const int waves = NG < kNumCUs * 8 ? NG : kNumCUs * 8;
    return (waves + 3) / 4;
}

// (L, U) of the fast path for C chunks per row, or 0 when it does not apply.
static int smallm_fast_shape(int C, int* L) {
    if (C == 16 || C == 32 || C == 48 || C == 64) {
        *L = 16;
        return C / 16;
    }
    if (C == 128 || C == 192) {
        *L = 64;
        return C / 64;
    }
    return 0;
}

template <int MT, int L>
static void launch_fast_mt(int U, dim3 g, dim3 b, size_t shm, hipStream_t s, const SmallMArgs& a) {
    switch (U) {
        case 1: smallm_fast_kernel<MT, L, 1><<<g, b, shm, s>>>(a); break;
        case 2: smallm_fast_kernel<MT, L, 2><<<g, b, shm, s>>>(a); break;
        case 3: smallm_fast_kernel<MT, L, 3><<<g, b, shm, s>>>(a); break;
        default: smallm_fast_kernel<MT, L, 4><<<g, b, shm, s>>>(a); break;
    }
}

template <int MT>
static void launch_fast(int L, int U, dim3 g, dim3 b, size_t shm, hipStream_t s,
                        const SmallMArgs& a) {
    if (L == 16)
        launch_fast_mt<MT, 16>(U, g, b, shm, s, a);
    else
        launch_fast_mt<MT, 64>(U, g, b, shm, s, a);
}

template <int MT>
static void launch_mt(bool lds, dim3 g, dim3 b, size_t shm, hipStream_t s,
                      const SmallMArgs& a) {
    if (lds)
        smallm_kernel<MT, true><<<g, b, shm, s>>>(a);
    else
        smallm_kernel<MT, false><<<g, b, 0, s>>>(a);
}

// More than 64 KB of dynamic LDS needs the kernel's limit raised, once per
// device (setting it again is harmless, so racing threads are benign; a
// failure shows as the launch's error).
template <int NB, bool HAD, bool G32>
static void launch_smq_nb(dim3 g, dim3 b, size_t shm, hipStream_t s, const SmqArgs& a) {
    static bool raised[64] = {};
    int dev = 0;
    if (shm > 64 * 1024 && hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64 &&
        !raised[dev]) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&smallm_mfma_kernel<NB, HAD, G32>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmqLds);
        raised[dev] = true;
    }
    smallm_mfma_kernel<NB, HAD, G32><<<g, b, shm, s>>>(a);
}

template <bool HAD, bool G32>
static void launch_smq(int NB, dim3 g, dim3 b, size_t shm, hipStream_t s, const SmqArgs& a) {
    switch (NB) {
        case 1: launch_smq_nb<1, HAD, G32>(g, b, shm, s, a); break;
        case 2: launch_smq_nb<2, HAD, G32>(g, b, shm, s, a); break;
        case 3: launch_smq_nb<3, HAD, G32>(g, b, shm, s, a); break;
        default: launch_smq_nb<4, HAD, G32>(g, b, shm, s, a); break;
    }
}

int launch_smallm(const void* packed, int N, int K, int group, int M,
                  const uint16_t* X, int ldx, void* Y, int ldy, int ydt,
                  hipStream_t s, int had_block) {
    if (had_block && (had_block != 512 || K % 512 != 0 || !smallm_mfma_applies(M, N, K, group)))
        return hip_fail(hipErrorInvalidValue, "smallM: fused transform needs the matrix-core path");
    SmallMArgs a;
    a.codes = static_cast<const u32x4*>(packed);
    a.scales = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(packed) +
                                                 scale_offset(N, K));
    a.X = X;
    a.Y = Y;
    a.N = N;
    a.C = K / 32;
    a.G = K / group;
    a.gshift = ilog2(group / 32);
    a.M = M;
    a.ldx = ldx;
    a.ldy = ldy;
    a.ydt = ydt;
    a.K = K;
    const SmqPlan mp = plan_smq(M, N, K, group);
    if (smallm_mfma_applies(M, N, K, group)) {   // W4_FORCE_PATH smallm_valu: vector ALU only
        SmqArgs b;
        b.codes = static_cast<const uint8_t*>(packed);
        b.scales = a.scales;
        b.X = X;
        b.Y = Y;
        b.N = N;
        b.K = K;
        b.G = K / group;
        b.group = group;
        b.M = M;
        b.ldx = ldx;
        b.ldy = ldy;
        b.ydt = ydt;
        b.RG = mp.RG;
        b.KS = mp.KS;
        b.had = had_block;
        b.hscale = (float)(1.0 / __builtin_sqrt(512.0));   // as the transform kernel
        const dim3 g(mp.grid), bl(64 * mp.RG * mp.KS);
        if (group == 32) {
            if (had_block)
                launch_smq<true, true>(mp.NB, g, bl, mp.lds, s, b);
            else
                launch_smq<false, true>(mp.NB, g, bl, mp.lds, s, b);
        } else {
            if (had_block)
                launch_smq<true, false>(mp.NB, g, bl, mp.lds, s, b);
            else
                launch_smq<false, false>(mp.NB, g, bl, mp.lds, s, b);
        }
        return hip_fail(hipGetLastError(), "smallM launch");
    }
    const size_t shm = smallm_lds(M, K);
    const bool lds = shm <= kSmLdsMax;
    int L = 16;
    const int U = smallm_fast_shape(K / 32, &L);
    if (lds && U > 0) {
        const dim3 g(smallm_grid(N, 64 / L)), b(256);
        if (M <= 4)
            launch_fast<4>(L, U, g, b, shm, s, a);
        else if (M <= 8)
            launch_fast<8>(L, U, g, b, shm, s, a);
        else
            launch_fast<16>(L, U, g, b, shm, s, a);
        return hip_fail(hipGetLastError(), "smallM launch");
    }
    const dim3 g(smallm_grid(N)), b(256);
    if (M <= 4)
        launch_mt<4>(lds, g, b, shm, s, a);
    else if (M <= 8)
        launch_mt<8>(lds, g, b, shm, s, a);
    else
        launch_mt<16>(lds, g, b, shm, s, a);
    return hip_fail(hipGetLastError(), "smallM launch");
}

void describe_smallm(int M, int N, int K, int group, char* buf, size_t len) {
    const SmqPlan mp = plan_smq(M, N, K, group);
    if (smallm_mfma_applies(M, N, K, group)) {
        snprintf(buf, len, "smallm mfma 16x16x32 rows %d x slices %d (K %d each) grid=%d",
                 16 * mp.RG, mp.KS, 128 * mp.NB, mp.grid);
        return;
    }
    const size_t shm = smallm_lds(M, K);
    int L = 16;
    const int U = smallm_fast_shape(K / 32, &L);
    if (shm <= kSmLdsMax && U > 0) {
        snprintf(buf, len, "smallm MT=%d L=%d U=%d x=lds grid=%d", M <= 4 ? 4 : (M <= 8 ? 8 : 16),
                 L, U, smallm_grid(N, 64 / L));
        return;
    }
    snprintf(buf, len, "smallm MT=%d L=%d x=%s grid=%d", M <= 4 ? 4 : (M <= 8 ? 8 : 16),
             kSmL, shm <= kSmLdsMax ? "lds" : "global", smallm_grid(N));
}

}  // namespace w4
