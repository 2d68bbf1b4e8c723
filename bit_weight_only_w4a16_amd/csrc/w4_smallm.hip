// w4_smallm.hip -- W4A16 product for 2 <= M <= 16 activation rows.
//
// [P2] "fastgemma -- Gemma 4 E2B, CPU-only, AMX INT8 / AVX-512 VNNI", section
// "Why AMX for GEMM but not for attention": a weight GEMM reuses each weight
// byte across all M rows.  Each packed chunk is loaded and decoded to bf16
// operand pairs once, then multiplied by every activation row.
//
// Work split as in the batch-1 GEMV: 16 lanes share a weight row (lane l owns
// chunks l, l + 16, ...), a wave covers 4 rows per step.  The activation rows
// and their per-chunk offset terms (136 * sum of the chunk's activations) are
// staged once per workgroup in LDS when they fit; otherwise they are read
// through the cache and the offset term is formed on the fly.  At this size
// the kernel is bound by vector ALU work (one dot2 per two codes per row).
#include <cstdio>

#include "w4_dispatch.h"

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
    float* xbs = reinterpret_cast<float*>(smem + (size_t)a.M * a.K * 2);  // [M][C]
    if (XLDS) {
        const int vec_per_row = a.K / 8;  // u32x4 per row
        for (int i = threadIdx.x; i < a.M * vec_per_row; i += blockDim.x) {
            const int m = i / vec_per_row, v = i % vec_per_row;
            const u32x4 val = reinterpret_cast<const u32x4*>(a.X + (size_t)m * a.ldx)[v];
            reinterpret_cast<u32x4*>(xs)[i] = val;
        }
        __syncthreads();
        for (int i = threadIdx.x; i < a.M * a.C; i += blockDim.x) {
            const int m = i / a.C, c = i % a.C;
            uint32_t xr[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) xr[j] = xs[(size_t)m * (a.K / 2) + c * 16 + j];
            xbs[i] = chunk_bias(xr);
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
                const float s = bf16_to_f32(a.scales[(size_t)n * a.G + (c >> a.gshift)]);
                uint32_t d[16];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        d[4 * w + j] = ((q[w] >> (4 * j)) & kPairMask) | kMagic;
                }
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    if (m < a.M) {
                        uint32_t xr[16];
                        float xb;
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
                            xb = xbs[m * a.C + c];
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
                            xb = chunk_bias(xr);
                        }
                        // same chain order as chunk_bias (exact zero for code 8)
                        float d0 = 0.f, d1 = 0.f;
#pragma unroll
                        for (int i = 0; i < 16; i += 2) {
                            d0 = dot2(d[i], xr[i], d0);
                            d1 = dot2(d[i + 1], xr[i + 1], d1);
                        }
                        acc[m] = fmaf(s, (d0 + d1) - xb, acc[m]);
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

static size_t smallm_lds(int M, int K) {
    return (size_t)M * K * 2 + (size_t)M * (K / 32) * 4;
}

static int smallm_grid(int N) {
    const int NG = (N + 3) / 4;
    const int waves = NG < kNumCUs * 8 ? NG : kNumCUs * 8;
    return (waves + 3) / 4;
}

template <int MT>
static void launch_mt(bool lds, dim3 g, dim3 b, size_t shm, hipStream_t s,
                      const SmallMArgs& a) {
    if (lds)
        smallm_kernel<MT, true><<<g, b, shm, s>>>(a);
    else
        smallm_kernel<MT, false><<<g, b, 0, s>>>(a);
}

int launch_smallm(const void* packed, int N, int K, int group, int M,
                  const uint16_t* X, int ldx, void* Y, int ldy, int ydt,
                  hipStream_t s) {
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
    const size_t shm = smallm_lds(M, K);
    const bool lds = shm <= kSmLdsMax;
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
    (void)group;
    const size_t shm = smallm_lds(M, K);
    snprintf(buf, len, "smallm MT=%d L=%d x=%s grid=%d", M <= 4 ? 4 : (M <= 8 ? 8 : 16),
             kSmL, shm <= kSmLdsMax ? "lds" : "global", smallm_grid(N));
}

}  // namespace w4
