// w4_fwht.hip -- blockwise fast Walsh-Hadamard transform of activation rows.
//
// [P2] "fastgemma -- Gemma 4 E2B, CPU-only, AMX INT8 / AVX-512 VNNI", section
// "What is in the file": weights are rotated along K by an orthogonal
// Hadamard matrix and the activation gets a fast Walsh-Hadamard transform at
// run time, which leaves the product unchanged.  Here: Sylvester order,
// orthonormal scale block^-1/2, contiguous blocks along K.
//
// One wave transforms one (row, block).  With E = block / 64 elements per lane
// (E >= 1), lane l holds elements l*E .. l*E + E - 1: butterfly spans below E
// stay inside a lane, spans h >= E pair lane l with lane l ^ (h / E).  fp32
// arithmetic, one scaling at the end, bf16 result rounded to nearest even.
#include "w4_dispatch.h"
#include "w4_fwht.h"

namespace w4 {

template <int E>
__global__ __launch_bounds__(256) void fwht_kernel(const uint16_t* X, int ldx,
                                                   uint16_t* Xo, int ldo, int M, int K,
                                                   int block, float scale) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nb = K / block;
    const long job = (long)blockIdx.x * (blockDim.x >> 6) + wave;
    if (job >= (long)M * nb) return;
    const int m = (int)(job / nb);
    const int b = (int)(job % nb);
    const int lanes = block / E;  // <= 64
    const bool active = lane < lanes;
    const uint16_t* src = X + (size_t)m * ldx + (size_t)b * block + (size_t)lane * E;
    float v[E];
    if (E >= 8) {
        // E contiguous bf16 per lane, 16-byte aligned (ldx % 8 == 0)
#pragma unroll
        for (int h = 0; h < E / 8; ++h) {
            const u32x4 w = reinterpret_cast<const u32x4*>(src)[h];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[8 * h + 2 * i] = __uint_as_float(w[i] << 16);
                v[8 * h + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = active ? bf16_to_f32(src[e]) : 0.f;
    }
    fwht_block<E>(v, lane, lanes);
    if (active) {
        uint16_t* dst = Xo + (size_t)m * ldo + (size_t)b * block + (size_t)lane * E;
        if (E >= 8) {
#pragma unroll
            for (int h = 0; h < E / 8; ++h) {
                u32x4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    w[i] = f32_to_bf16_rne(v[8 * h + 2 * i] * scale) |
                           (f32_to_bf16_rne(v[8 * h + 2 * i + 1] * scale) << 16);
                reinterpret_cast<u32x4*>(dst)[h] = w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) dst[e] = (uint16_t)f32_to_bf16_rne(v[e] * scale);
        }
    }
}

int launch_fwht(const uint16_t* X, int ldx, uint16_t* Xo, int ldo, int M, int K,
                int block, hipStream_t s) {
    const long jobs = (long)M * (K / block);
    const dim3 b(256), g((unsigned)((jobs + 3) / 4));
    // block^-1/2 in double, rounded once to fp32 (exact for even powers of 2)
    const float scale = (float)(1.0 / __builtin_sqrt((double)block));
    switch (block <= 64 ? 1 : block / 64) {
        case 1: fwht_kernel<1><<<g, b, 0, s>>>(X, ldx, Xo, ldo, M, K, block, scale); break;
        case 2: fwht_kernel<2><<<g, b, 0, s>>>(X, ldx, Xo, ldo, M, K, block, scale); break;
        case 4: fwht_kernel<4><<<g, b, 0, s>>>(X, ldx, Xo, ldo, M, K, block, scale); break;
        case 8: fwht_kernel<8><<<g, b, 0, s>>>(X, ldx, Xo, ldo, M, K, block, scale); break;
        default: fwht_kernel<16><<<g, b, 0, s>>>(X, ldx, Xo, ldo, M, K, block, scale); break;
    }
    return hip_fail(hipGetLastError(), "fwht launch");
}

}  // namespace w4
