// w4_gather.hip -- rows of a packed 4-bit table, dequantized on the GPU.
//
// [P1] "Gemma 4 E2B on a 4 GB GPU with plain PyTorch, faster than llama.cpp",
// step 2 "Keep the Vocabulary Tables in 4-Bit": the token-embedding table
// (one copy that also serves as the output layer) and the per-layer input
// table (35 x 256 values per token) stay as 4-bit codes with a 16-bit step
// per group, and the per-token lookup runs on the GPU.  A looked-up row is
// the dequantized row (code - 8) * scale, which fp32 holds exactly; a bf16
// output is that value rounded to nearest even.
//
// The table is in the device layout every kernel reads (w4_pack), so the
// embedding lookup and the output layer's GEMV share one copy.
#include "w4_dispatch.h"

namespace w4 {

// One thread per device word (8 elements) of an output row: one 4-byte code
// load and one scale; consecutive threads take consecutive words of a row,
// so a wave's code loads are 256 contiguous bytes and its stores 1 KB (bf16)
// or 2 KB (fp32) contiguous.  An id outside [0, N) reads nothing and writes
// quiet NaNs.
template <int YDT>
__global__ __launch_bounds__(256) void gather_kernel(const uint32_t* __restrict__ words,
                                                     const uint16_t* __restrict__ scales,
                                                     int N, int W, int G, int gshift,
                                                     const int32_t* __restrict__ ids,
                                                     int B, void* __restrict__ Y, int ldy) {
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (long long)B * W) return;
    const int b = (int)(t / W);
    const int d = (int)(t - (long long)b * W);   // word of the row: elements 8d .. 8d + 7
    const int id = gload(ids + b);
    const bool valid = id >= 0 && id < N;

    // element 8d + 2i at bits [4i, 4i + 4), element 8d + 2i + 1 at bits
    // [16 + 4i, 20 + 4i)
    float v[8];
    if (valid) {
        const uint32_t w = gload(words + (size_t)id * W + d);
        const float s = bf16_to_f32(gload(scales + (size_t)id * G + ((d >> 2) >> gshift)));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = (float)((int)((w >> (4 * i)) & 15u) - 8) * s;
            v[2 * i + 1] = (float)((int)((w >> (16 + 4 * i)) & 15u) - 8) * s;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = __builtin_nanf("");
    }

    if (YDT == W4_F32) {
        u32x4* y = reinterpret_cast<u32x4*>(static_cast<float*>(Y) + (size_t)b * ldy + 8 * d);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            u32x4 o;
            o[0] = __float_as_uint(v[4 * j + 0]);
            o[1] = __float_as_uint(v[4 * j + 1]);
            o[2] = __float_as_uint(v[4 * j + 2]);
            o[3] = __float_as_uint(v[4 * j + 3]);
            gstore(y + j, o);
        }
    } else {
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = valid ? (f32_to_bf16_rne(v[2 * j]) | (f32_to_bf16_rne(v[2 * j + 1]) << 16))
                         : 0x7FC07FC0u;
        gstore(reinterpret_cast<u32x4*>(static_cast<uint16_t*>(Y) + (size_t)b * ldy + 8 * d), o);
    }
}

int launch_gather(const void* packed, int N, int K, int group, const int32_t* ids, int B,
                  void* Y, int ldy, int ydt, hipStream_t s) {
    if (B == 0) return W4_OK;
    const int W = K / 8;   // device words per row
    const uint32_t* words = static_cast<const uint32_t*>(packed);
    const uint16_t* scales = reinterpret_cast<const uint16_t*>(
        static_cast<const uint8_t*>(packed) + scale_offset(N, K));
    const long long work = (long long)B * W;
    const dim3 grid((unsigned)((work + 255) / 256)), block(256);
    if (ydt == W4_F32)
        gather_kernel<W4_F32><<<grid, block, 0, s>>>(words, scales, N, W, K / group,
                                                      ilog2(group / 32), ids, B, Y, ldy);
    else
        gather_kernel<W4_BF16><<<grid, block, 0, s>>>(words, scales, N, W, K / group,
                                                       ilog2(group / 32), ids, B, Y, ldy);
    return hip_fail(hipGetLastError(), "gather launch");
}

}  // namespace w4
