// w4_quant.hip -- rotate-and-quantize: dense weights -> the packed device layout.
//
// [P2] "fastgemma -- Gemma 4 E2B, CPU-only, AMX INT8 / AVX-512 VNNI", section
// "What is in the file": every linear weight is rotated along K by an
// orthogonal Hadamard matrix, W' = W H^T, and stored as int4 with one scale
// per group; with the run-time transform of the activation (w4_fwht) the
// product is unchanged, and rows with outliers quantize with less error.
// The page gives no scale rule.  Rule used: symmetric per group,
//   s = bf16(max|w'| / 7),  q = clamp(round_half_even(w' / s), -8, 7),
//   code = q + 8  (s = 0 and code 8 for an all-zero group),
// every step in fp32, so that the codes are a deterministic function of the
// fp32 rotated weights.
//
// One wave per (row, 512-element span): lane l holds elements 8l .. 8l+7,
// exactly one 32-bit code word.  The Hadamard butterflies run in increasing
// span order, spans 1, 2, 4 inside a lane and 8 .. block/2 across lanes
// (partner lane ^ (span / 8)), then one fp32 scaling; the group maximum is a
// cross-lane max over the group's group/8 lanes.
#include "w4_dispatch.h"

namespace w4 {

template <bool BF16IN>
__global__ __launch_bounds__(256) void quant_kernel(const void* __restrict__ W, int ldw, int N,
                                                    int K, int group, int block, float hscale,
                                                    uint32_t* __restrict__ codes,
                                                    uint16_t* __restrict__ scales) {
    const int lane = threadIdx.x & 63;
    const int spans = (K + 511) / 512;
    const long long job = (long long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (job >= (long long)N * spans) return;
    const int n = (int)(job / spans);
    const int k0 = (int)(job - (long long)n * spans) * 512 + 8 * lane;
    const bool active = k0 < K;  // K % 32 == 0: a group is all active or all idle

    float v[8];
    if (active) {
        if (BF16IN) {
            const u32x4 w = gload(reinterpret_cast<const u32x4*>(
                static_cast<const uint16_t*>(W) + (size_t)n * ldw + k0));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = __uint_as_float(w[i] << 16);
                v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
            }
        } else {
            const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(W) +
                                                            (size_t)n * ldw + k0);
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

    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
    for (int d = 1; d < group / 8; d *= 2) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
    const uint32_t sb = f32_to_bf16_rne(amax / 7.0f);
    const float sf = bf16_to_f32(sb);

    // device word: element 2i at bits [4i, 4i+4), element 2i+1 at [16+4i, 20+4i)
    uint32_t word = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float q = 0.f;
        if (sf != 0.f) q = fminf(fmaxf(__builtin_rintf(v[e] / sf), -8.f), 7.f);
        const uint32_t code = (uint32_t)((int)q + 8);
        word |= code << ((e & 1) ? 16 + 4 * (e >> 1) : 4 * (e >> 1));
    }
    if (active) {
        gstore(codes + (size_t)n * (K / 8) + k0 / 8, word);
        if (lane % (group / 8) == 0)
            gstore(scales + (size_t)n * (K / group) + k0 / group, (uint16_t)sb);
    }
}

int launch_quantize(const void* W, int wdt, int ldw, int N, int K, int group, int block,
                    void* packed, hipStream_t s) {
    uint32_t* codes = static_cast<uint32_t*>(packed);
    uint16_t* scales =
        reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(packed) + scale_offset(N, K));
    const long long jobs = (long long)N * ((K + 511) / 512);
    const dim3 b(256), g((unsigned)((jobs + 3) / 4));
    // block^-1/2 in double, rounded once to fp32
    const float hscale = block ? (float)(1.0 / __builtin_sqrt((double)block)) : 1.f;
    if (wdt == W4_BF16)
        quant_kernel<true><<<g, b, 0, s>>>(W, ldw, N, K, group, block, hscale, codes, scales);
    else
        quant_kernel<false><<<g, b, 0, s>>>(W, ldw, N, K, group, block, hscale, codes, scales);
    return hip_fail(hipGetLastError(), "quantize launch");
}

}  // namespace w4
