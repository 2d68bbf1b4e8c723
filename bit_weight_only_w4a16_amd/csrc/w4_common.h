// w4_common.h -- internal helpers shared by the library's translation units.
//
// Decode scheme (gfx950).  A code c in 0..15 placed in the low mantissa bits
// of the bf16 pattern 0x4300 (= 128.0) is the bf16 number 128 + c, exactly:
// bf16 has 7 stored mantissa bits and the spacing of bf16 numbers in
// [128, 256) is 1.  The device layout puts the codes of elements 2j and 2j+1
// of an 8-element word at bits [4j, 4j+4) and [16+4j, 20+4j), so one shift and
// one and-or turn a word into a bf16 pair (128 + c_2j, 128 + c_2j+1) that
// v_dot2_f32_bf16 multiplies by the activation pair (x_2j, x_2j+1) with fp32
// accumulation.  Products of two bf16 numbers are exact in fp32.  The offset
// is removed once per 32-element chunk: sum (128 + c) x - 136 sum x
// = sum (c - 8) x, the offset-binary value of the pages' decode
// ([P1] "Gemma 4 E2B on a 4 GB GPU with plain PyTorch, faster than
// llama.cpp", paragraph on the w4gemv.py kernel: each 4-bit value becomes the
// exact float (value - 8)).  For a one-hot activation the result is exactly
// (c - 8) * scale.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/w4a16.h"

namespace w4 {

// ------------------------------------------------------------ host errors --
void set_error(const char* fmt, ...);
int fail(int status, const char* fmt, ...);
int hip_fail(hipError_t e, const char* what);

// ------------------------------------------------------------------ layout --
constexpr size_t kAlign = 256;
__host__ __device__ inline size_t align_up(size_t v, size_t a) {
    return (v + a - 1) / a * a;
}
// Byte offset of the scales inside a packed buffer.
__host__ __device__ inline size_t scale_offset(int N, int K) {
    return align_up((size_t)N * (size_t)K / 2, kAlign);
}
__host__ __device__ inline size_t packed_bytes(int N, int K, int group) {
    return scale_offset(N, K) +
           align_up((size_t)N * (size_t)(K / group) * 2, kAlign);
}

// Canonical word (element j at bits [4j, 4j+4)) -> device word (even elements
// in the low half, odd elements in the high half).
__host__ __device__ inline uint32_t word_to_device(uint32_t w) {
    uint32_t out = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        out |= ((w >> (8 * j)) & 0xFu) << (4 * j);            // element 2j
        out |= ((w >> (8 * j + 4)) & 0xFu) << (16 + 4 * j);   // element 2j+1
    }
    return out;
}
__host__ __device__ inline uint32_t word_from_device(uint32_t d) {
    uint32_t out = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        out |= ((d >> (4 * j)) & 0xFu) << (8 * j);
        out |= ((d >> (16 + 4 * j)) & 0xFu) << (8 * j + 4);
    }
    return out;
}

inline int ilog2(int v) {
    int r = 0;
    while ((1 << r) < v) ++r;
    return r;
}

// ------------------------------------------------------------------ device --
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kPairMask = 0x000F000Fu;
constexpr uint32_t kMagic = 0x43004300u;      // bf16 pair (128, 128)
constexpr uint32_t kOffsetPair = 0x43084308u; // bf16 pair (136, 136)

__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
    return __uint_as_float(h << 16);
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;  // NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c,
                                           false);
}

// The decode constants as opaque VGPR values: with the mask and the magic in
// registers the compiler selects one v_and_or_b32 per operand pair (gfx9 VOP3
// encodings take no literal constants).
struct DecodeConsts {
    uint32_t mask, magic, offset;
};
__device__ __forceinline__ DecodeConsts decode_consts() {
    DecodeConsts k;
    asm volatile("v_mov_b32 %0, 0xf000f" : "=v"(k.mask));
    asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(k.magic));
    asm volatile("v_mov_b32 %0, 0x43084308" : "=v"(k.offset));
    return k;
}

// Operand pair j of device word w: bf16 (128 + c_2j, 128 + c_2j+1).
__device__ __forceinline__ uint32_t decode_pair(uint32_t w, int j, const DecodeConsts& k) {
    return ((w >> (4 * j)) & k.mask) | k.magic;
}

// One 32-element chunk: sum over the chunk of (128 + c_k) * x_k, with q the
// chunk's 4 device words and xr its 16 bf16 activation pairs (pair i holds
// elements 2i, 2i+1).  Two accumulation chains (even / odd pairs), each
// started at zero, in the same order as chunk_bias: for a chunk whose codes
// are all 8 the decoded pairs equal the offset pair (136, 136), both
// computations round identically, and the chunk contributes exactly zero.
__device__ __forceinline__ float chunk_dot(u32x4 q, const uint32_t* xr,
                                           const DecodeConsts& k) {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t w = q[d];
        a0 = dot2(decode_pair(w, 0, k), xr[4 * d + 0], a0);
        a1 = dot2(decode_pair(w, 1, k), xr[4 * d + 1], a1);
        a0 = dot2(decode_pair(w, 2, k), xr[4 * d + 2], a0);
        a1 = dot2(decode_pair(w, 3, k), xr[4 * d + 3], a1);
    }
    return a0 + a1;
}

// 136 * sum of the chunk's 32 activations (the bias of chunk_dot plus the
// code offset 8), fp32, accumulated exactly like chunk_dot.
__device__ __forceinline__ float chunk_bias(const uint32_t* xr) {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
        a0 = dot2(kOffsetPair, xr[i], a0);
        a1 = dot2(kOffsetPair, xr[i + 1], a1);
    }
    return a0 + a1;
}

// Sum over groups of L consecutive lanes (L in 8, 16, 32, 64) with DPP moves
// inside each 16-lane row and swizzles across rows; every lane of a group
// ends with the group's total.  The order is fixed, so results are bitwise
// deterministic.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over each 16-lane row; every lane of the row ends with the row's total
// (the same fixed order as group_sum<16>).
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_mov<0x128>(v);  // row_ror:8
    v += dpp_mov<0x124>(v);  // row_ror:4
    v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
    return v;
}

// DPP row broadcast (row_bcast:15 = 0x142, row_bcast:31 = 0x143) into the
// rows of ROWMASK; the other rows get 0.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_row_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWMASK, 0xF, false));
}

template <int L>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(L == 8 || L == 16 || L == 32 || L == 64, "group size");
    if (L >= 16) {
        v += dpp_mov<0x128>(v);  // row_ror:8
        v += dpp_mov<0x124>(v);  // row_ror:4
    } else {
        v += dpp_mov<0x141>(v);  // row_half_mirror
    }
    v += dpp_mov<0x4E>(v);       // quad_perm [2,3,0,1]
    v += dpp_mov<0xB1>(v);       // quad_perm [1,0,3,2]
    if (L >= 32) v += __shfl_xor(v, 16, 64);
    if (L >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// Global-memory accesses through pointers typed as global.  A pointer that
// was read out of device memory (an op table) is generic to the compiler,
// and generic (flat) loads hold the LDS counter as well as the vector-memory
// counter: the wait before any LDS or cross-lane result would then also wait
// for every weight load in flight.  Every operand these helpers touch is in
// global memory.
template <typename T>
using global_t = __attribute__((address_space(1))) T;

template <typename T>
__device__ __forceinline__ T nt_load(const T* p) {
    return __builtin_nontemporal_load((const global_t<T>*)p);
}

template <typename T>
__device__ __forceinline__ T gload(const T* p) {
    return *(const global_t<T>*)p;
}

template <typename T>
__device__ __forceinline__ void gstore(T* p, T v) {
    *(global_t<T>*)p = v;
}

// Scales are read as the aligned dword that holds them (rows of an even
// number of groups keep every row's scales dword-aligned); the bf16 is moved
// into the high half of an fp32 with one byte permute at its use.  A 16-bit
// load would need a conversion right after it, and the compiler places such
// a conversion where it reuses the load's register, waiting for the load
// there -- before the next row group's loads are issued.
constexpr uint32_t kScaleSelLo = 0x01000C0Cu;  // bytes 1,0 -> 3,2; zeros below
constexpr uint32_t kScaleSelHi = 0x03020C0Cu;  // bytes 3,2 -> 3,2; zeros below

__device__ __forceinline__ float scale_from_word(uint32_t w, uint32_t sel) {
    return __uint_as_float(__builtin_amdgcn_perm(0u, w, sel));
}

__device__ __forceinline__ void store_out(void* y, size_t i, float v, int ydt) {
    if (ydt == W4_BF16)
        gstore(static_cast<uint16_t*>(y) + i, (uint16_t)f32_to_bf16_rne(v));
    else
        gstore(static_cast<float*>(y) + i, v);
}

}  // namespace w4
