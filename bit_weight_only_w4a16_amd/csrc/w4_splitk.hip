// w4_splitk.hip -- W4A16 product for 2..32 activation rows on the matrix
// cores, K split across the four waves of a workgroup.
//
// [P2] "fastgemma -- Gemma 4 E2B, CPU-only, AMX INT8 / AVX-512 VNNI", section
// "Why AMX for GEMM but not for attention": a weight GEMM reuses each weight
// byte across all M rows.  At a few dozen rows the product is still close to
// its weight stream (N K / 2 bytes), so this kernel is built for streaming:
//
// - a workgroup owns 48 weight rows (three 16-row MFMA tiles) and every
//   activation row (MF = 1 or 2 tiles of 16 rows); its four waves, one per
//   SIMD, take one quarter of K each, so a 12288-row matrix is one
//   workgroup per CU;
// - a wave issues all of its code words (straight into registers) and all
//   of its activation blocks (global-to-LDS DMA into its own LDS region) at
//   its start, so the launch's whole weight stream is in flight at once.
//   Activations are read by every workgroup (from L2 after the first touch);
//   the DMA reads them as whole 256-byte row spans, four rows per load,
//   where loads in the MFMA operand layout would touch 16 rows per 16
//   lanes (measured: 11.0 against 8.7 us at 64 rows, 7.8 against 6.7 at 32);
// - waits: group 32 starts each block once its own activations and codes
//   are in, groups 256 and 512 once every first load is in (each faster for
//   its group, by 0.5-0.7 and 0.2-0.3 us);
// - the four slice sums meet in LDS and are added in slice order 0..3, so
//   the result is deterministic.
//
// MFMA v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8(l/16)+j],
// B[8(l/16)+j][l%16] and D[4(l/16)+r][l%16].  Codes decode to the exact bf16
// values 16 (c - 8) (w4_common.h), each group's product is scaled by s / 16.
// Groups of 256 and 512: lane group l/16 loads chunk l/16 of each 128-K
// block of its row (16 bytes) and uses word t in MFMA step t, the activations
// read with the same K permutation; a block lies inside one group, whose sum
// is scaled when the group (or the slice) ends.  Group 32: step t must cover
// exactly chunk t, one group, so the loaded words are transposed 4 x 4 across
// the lane groups (lane group l/16 then holds word 4t + l/16) and every step
// is scaled on its own.
#include <cstdio>

#include "w4_config.h"
#include "w4_dispatch.h"
#include "w4_ring.h"

namespace w4 {

constexpr int kSkWaves = 4;   // K slices per workgroup (one wave per SIMD)
constexpr int kSkNF = 3;      // 16-row weight tiles per workgroup
constexpr int kSkRows = 16 * kSkNF;

struct SkArgs {
    const uint8_t* codes;    // N x K/2 bytes (device words)
    const uint16_t* scales;  // N x G bf16
    const uint16_t* X;       // M x K bf16, row stride ldx
    void* Y;
    int N, K, G, group, M, ldx, ldy, ydt;
};

// LDS: each wave stages all of its activation blocks (128 K each, 16 MF
// rows x 256 bytes; at most 4 blocks of 8 KB per wave).
__host__ __device__ constexpr int sk_lds_bytes(int MF, int NB) {
    return kSkWaves * NB * 16 * MF * 256;
}

typedef __bf16 sk_bf16x8 __attribute__((ext_vector_type(8)));
typedef float sk_f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ sk_f32x4 sk_mfma(u32x4 a, u32x4 b, sk_f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(sk_bf16x8, a),
                                                   __builtin_bit_cast(sk_bf16x8, b), c, 0, 0, 0);
}

// 4 x 4 word transpose across the lane groups: lane group r holds words
// 4r .. 4r + 3 of a block, afterwards word 4t + r in position t.  Step 1
// swaps across lane groups r, r ^ 1 (16 lanes apart), step 2 across r, r ^ 2.
__device__ __forceinline__ u32x4 sk_transpose(u32x4 v, int lk) {
    const bool b0 = (lk & 1) != 0, b1 = (lk & 2) != 0;
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
    return v;
}

// Wait until block b's activation DMA has landed: NB blocks of DB loads,
// followed by W code-word loads.  b is a constant once the block loop is
// unrolled, so one wait remains.
template <int NB, int DB, int W, int I = 0>
__device__ __forceinline__ void sk_wait_block(int b) {
    if constexpr (I < NB) {
        if (b == I)
            ring::wait_vm<(NB - 1 - I) * DB + W>();
        else
            sk_wait_block<NB, DB, W, I + 1>(b);
    }
}

// MF activation tiles, NB 128-K blocks per wave.
template <int MF, int NB, bool G32>
__global__ __launch_bounds__(64 * kSkWaves) __attribute__((amdgpu_waves_per_eu(1, 1)))
void splitk_kernel(SkArgs a) {
    constexpr int NF = kSkNF;
    // group 32 starts each block once its own operands are in (measured
    // faster: 6.5 against 7.2 us at 8 rows); groups 256 and 512 start once
    // every first load is in (5.3 against 5.5 us at 16 rows, 6.7 against
    // 7.0 at 32)
    constexpr bool PRECISE = G32;
    constexpr int DB = 4 * MF;                  // DMA loads per activation block
    constexpr int AB = 16 * MF * 256;           // bytes of one activation block
    extern __shared__ __align__(16) uint8_t sk_lds[];
    const int lane = threadIdx.x & 63;
    const int ks = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15, lk = lane >> 4;
    const int n0 = blockIdx.x * kSkRows;
    const int k0 = ks * 128 * NB;

    // this lane's weight rows (rows past N read row N - 1, never stored)
    const uint8_t* crow[NF];
    int srow[NF];
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) {
        const int n = min(n0 + 16 * nf + li, a.N - 1);
        crow[nf] = a.codes + (size_t)n * (a.K / 2) + k0 / 2 + 16 * lk;
        srow[nf] = n * a.G;
    }

    // Activation blocks go to this wave's own LDS region by DMA, one
    // 16-byte piece per lane, 4 rows (1 KB) per load; piece p of row r sits
    // in slot p ^ (r % 16) of the row's 256 bytes, so that the 16 lanes of
    // an MFMA fragment read (16 rows, one piece each) hit 16 different slots
    // (conflict-free), while each load still reads whole 256-byte row spans.
    // Rows past M read row M - 1 (never stored).
    uint8_t* region = sk_lds + ks * NB * AB;
    const uint32_t region_lds = ring::lds_addr(region);
    const int dr = lane >> 4, dc = lane & 15;
    auto dma_block = [&](int b) {
#pragma unroll
        for (int j = 0; j < DB; ++j) {
            const int r = 4 * j + dr;
            const int m = min(r, a.M - 1);
            const uint32_t off = (uint32_t)m * (uint32_t)a.ldx * 2u + (uint32_t)(k0 + 128 * b) * 2u +
                                 16u * (uint32_t)(dc ^ (r & 15));
            ring::dma16(off, a.X, region_lds + b * AB + 1024 * j);
        }
    };
    // activation fragment of step t for tile mf: lane group lk's 8 elements
    // are piece 4 lk + t of the row's block (groups >= 128) or piece 4 t +
    // lk (group 32)
    auto frag = [&](int b, int mf, int t) {
        const int p = G32 ? 4 * t + lk : 4 * lk + t;
        return *reinterpret_cast<const u32x4*>(region + b * AB + (16 * mf + li) * 256 +
                                               16 * (p ^ li));
    };

    // Everything the wave reads is issued at its start.  The compiler's own
    // waits (for codes and scales) do not count the DMA loads, and would
    // wait for any issued after what they need, so with per-block waits
    // (group 32) the order is scales, activation blocks (DMA), code words;
    // otherwise code words, activation blocks, scales (measured 0.2-0.3 us
    // faster than scales first at 2..16 rows).
    uint32_t sw[NB][NF][G32 ? 2 : 1];
    uint32_t ssel[NB][NF];
    auto load_scales = [&]() {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int nf = 0; nf < NF; ++nf) {
                // groups of 32: the block's four scales as one 8-byte load;
                // otherwise the aligned dword that holds the block's group
                // scale
                if constexpr (G32) {
                    const u32x2 v = gload(reinterpret_cast<const u32x2*>(
                        a.scales + srow[nf] + (k0 + 128 * b) / 32));
                    sw[b][nf][0] = v[0];
                    sw[b][nf][1] = v[1];
                    ssel[b][nf] = 0;
                } else {
                    const int e = srow[nf] + (k0 + 128 * b) / a.group;
                    sw[b][nf][0] = gload(reinterpret_cast<const uint32_t*>(a.scales + (e & ~1)));
                    ssel[b][nf] = (e & 1) ? kScaleSelHi : kScaleSelLo;
                }
            }
        asm volatile("" ::: "memory");
    };
    u32x4 q[NB][NF];
    auto load_codes = [&]() {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int nf = 0; nf < NF; ++nf)
                q[b][nf] = nt_load(reinterpret_cast<const u32x4*>(crow[nf] + 64 * b));
        asm volatile("" ::: "memory");
    };
    if constexpr (PRECISE)
        load_scales();
    else
        load_codes();
#pragma unroll
    for (int b = 0; b < NB; ++b) dma_block(b);
    asm volatile("" ::: "memory");
    if constexpr (PRECISE)
        load_codes();
    else
        load_scales();

    const sk_f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    sk_f32x4 acc[MF][NF], tot[MF][NF];
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) {
            acc[mf][nf] = zero;   // (group 32 uses tot only)
            tot[mf][nf] = zero;
        }

#pragma unroll
    for (int b = 0; b < NB; ++b) {
        // block b's activations have landed (per block: at most the loads
        // issued after them are in flight; otherwise every load has, once)
        if constexpr (PRECISE)
            sk_wait_block<NB, DB, NB * NF>(b);
        else if (b == 0)
            ring::wait_vm<0>();
        asm volatile("" ::: "memory");
        if constexpr (G32) {
#pragma unroll
            for (int nf = 0; nf < NF; ++nf) q[b][nf] = sk_transpose(q[b][nf], lk);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                u32x4 x[MF];
#pragma unroll
                for (int mf = 0; mf < MF; ++mf) x[mf] = frag(b, mf, t);
#pragma unroll
                for (int nf = 0; nf < NF; ++nf) {
                    const u32x4 bv = decode_x16(q[b][nf][t]);
                    const uint32_t w = sw[b][nf][t >> 1];
                    const float s = __uint_as_float((t & 1) ? (w & 0xFFFF0000u) : (w << 16)) *
                                    0.0625f;
#pragma unroll
                    for (int mf = 0; mf < MF; ++mf) {
                        const sk_f32x4 p = sk_mfma(x[mf], bv, zero);
#pragma unroll
                        for (int r = 0; r < 4; ++r) tot[mf][nf][r] = fmaf(s, p[r], tot[mf][nf][r]);
                    }
                }
            }
        } else {
            // a group's first block starts its sums from zero
            const bool gstart = b == 0 || (k0 + 128 * b) % a.group == 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                u32x4 x[MF];
#pragma unroll
                for (int mf = 0; mf < MF; ++mf) x[mf] = frag(b, mf, t);
#pragma unroll
                for (int nf = 0; nf < NF; ++nf) {
                    const u32x4 bv = decode_x16(q[b][nf][t]);
                    if (t == 0 && gstart) {
#pragma unroll
                        for (int mf = 0; mf < MF; ++mf) acc[mf][nf] = sk_mfma(x[mf], bv, zero);
                    } else {
#pragma unroll
                        for (int mf = 0; mf < MF; ++mf)
                            acc[mf][nf] = sk_mfma(x[mf], bv, acc[mf][nf]);
                    }
                }
            }
            // the group (or this slice's part of it) ends with this block
            const bool gend = b == NB - 1 || (k0 + 128 * (b + 1)) % a.group == 0;
            if (gend) {
#pragma unroll
                for (int nf = 0; nf < NF; ++nf) {
                    const float s = scale_from_word(sw[b][nf][0], ssel[b][nf]) * 0.0625f;
#pragma unroll
                    for (int mf = 0; mf < MF; ++mf) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            tot[mf][nf][r] = fmaf(s, acc[mf][nf][r], tot[mf][nf][r]);
                    }
                }
            }
        }
    }

    // slice sums, each wave's in its own region, added in slice order; wave
    // w stores tiles w, w + 4, ...
    sk_f32x4* red = reinterpret_cast<sk_f32x4*>(sk_lds);
    constexpr int RS = NB * AB / 16;   // a region, in 16-byte units
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) red[ks * RS + (mf * NF + nf) * 64 + lane] = tot[mf][nf];
    __syncthreads();
    for (int p = ks; p < MF * NF; p += kSkWaves) {
        sk_f32x4 v = red[p * 64 + lane];
#pragma unroll
        for (int j = 1; j < kSkWaves; ++j) {
            const sk_f32x4 o = red[j * RS + p * 64 + lane];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] += o[r];
        }
        const int mf = p / NF, nf = p - mf * NF;
        const int n = n0 + 16 * nf + li;
        if (n < a.N) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 16 * mf + 4 * lk + r;
                if (m < a.M) store_out(a.Y, (size_t)m * a.ldy + n, v[r], a.ydt);
            }
        }
    }
}

struct SkPlan {
    bool ok;
    int MF, NB, grid;
};

// Applies to 2..32 rows (8..32 at group 32), groups 32, 256 and 512, K a
// multiple of 512 up to 2048 (a quarter of K, NB <= 4 blocks of 128, per
// wave), matrices of at least 128 workgroups of 48 rows, and activations
// addressable with 32-bit offsets (the DMA loads').  Measured at N = 12288,
// K = 1536 against the kernels these shapes took before: group 256 5.2-5.3 us
// at 2..16 rows (5.6-6.9 on the matrix-core small-M kernel), 6.2-6.7 us at
// 17..32 (8.3-8.4 on the DMA ring); group 32 6.5-6.7 us at 8..16 (7.2-8.1),
// 7.5-8.3 at 17..32 (10.2-10.3).  Below 8 rows of group 32 the vector-ALU
// small-M kernel is as fast or faster (4.9-5.8 us at 2..4), and from 33 rows
// on, with four activation tiles per workgroup (two 16 KB blocks in LDS per
// wave), this kernel measured 8.5-8.9 us at 64 rows against the DMA ring's
// 8.4.
static SkPlan plan_splitk(int M, int N, int K, int group, int ldx) {
    SkPlan p{};
    p.ok = false;
    // W4_FORCE_PATH no_splitk, or a path that names another kernel for the
    // shape (smallm_valu up to 16 rows, prefill_regs above)
    const unsigned force = config()->force;
    if (force & kForceNoSplitK) return p;
    if ((force & kForceSmallmValu) && M <= 16) return p;
    if ((force & kForcePrefillRegs) && M > 16) return p;
    if (M < (group == 32 ? 8 : 2) || M > 32) return p;
    if (group != 32 && group != 256 && group != 512) return p;
    if (K % 512 != 0 || K > 2048) return p;
    if (((size_t)(M - 1) * (size_t)ldx + (size_t)K) * 2 >= (1ull << 32)) return p;
    p.grid = (N + kSkRows - 1) / kSkRows;
    if (p.grid < kNumCUs / 2) return p;
    p.MF = M <= 16 ? 1 : 2;
    p.NB = K / 512;
    p.ok = true;
    return p;
}

bool splitk_applies(int M, int N, int K, int group, int ldx) {
    return plan_splitk(M, N, K, group, ldx).ok;
}

template <int MF, int NB, bool G32>
static void splitk_launch_one(dim3 g, hipStream_t s, const SkArgs& a) {
    constexpr int lds = sk_lds_bytes(MF, NB);
    if (lds > 64 * 1024)   // (setting it again is harmless)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&splitk_kernel<MF, NB, G32>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    splitk_kernel<MF, NB, G32><<<g, dim3(64 * kSkWaves), lds, s>>>(a);
}

template <int MF>
static void splitk_launch_mf(int NB, bool g32, dim3 g, hipStream_t s, const SkArgs& a) {
    switch (NB * 2 + (g32 ? 1 : 0)) {
        case 2: splitk_launch_one<MF, 1, false>(g, s, a); break;
        case 3: splitk_launch_one<MF, 1, true>(g, s, a); break;
        case 4: splitk_launch_one<MF, 2, false>(g, s, a); break;
        case 5: splitk_launch_one<MF, 2, true>(g, s, a); break;
        case 6: splitk_launch_one<MF, 3, false>(g, s, a); break;
        case 7: splitk_launch_one<MF, 3, true>(g, s, a); break;
        case 8: splitk_launch_one<MF, 4, false>(g, s, a); break;
        default: splitk_launch_one<MF, 4, true>(g, s, a); break;
    }
}

int launch_splitk(const void* packed, int N, int K, int group, int M, const uint16_t* X,
                  int ldx, void* Y, int ldy, int ydt, hipStream_t s) {
    const SkPlan p = plan_splitk(M, N, K, group, ldx);
    if (!p.ok) return fail(W4_ERR_UNSUPPORTED, "splitk: shape not supported");
    SkArgs a;
    a.codes = static_cast<const uint8_t*>(packed);
    a.scales = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(packed) +
                                                 scale_offset(N, K));
    a.X = X;
    a.Y = Y;
    a.N = N;
    a.K = K;
    a.G = K / group;
    a.group = group;
    a.M = M;
    a.ldx = ldx;
    a.ldy = ldy;
    a.ydt = ydt;
    const dim3 g(p.grid);
    const bool g32 = group == 32;
    if (p.MF == 1)
        splitk_launch_mf<1>(p.NB, g32, g, s, a);
    else
        splitk_launch_mf<2>(p.NB, g32, g, s, a);
    return hip_fail(hipGetLastError(), "splitk launch");
}

void describe_splitk(int M, int N, int K, int group, int ldx, char* buf, size_t len) {
    const SkPlan p = plan_splitk(M, N, K, group, ldx);
    snprintf(buf, len,
             "splitk mfma 16x16x32 rows %d x %d activation tiles, K split 4 ways (%d each) "
             "grid=%d",
             kSkRows, p.MF, K / kSkWaves, p.grid);
}

}  // namespace w4
