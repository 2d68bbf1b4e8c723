// w4_common.h -- internal helpers shared by the library's translation units.
//
// Exact decode ([P1] "Gemma 4 E2B on a 4 GB GPU with plain PyTorch, faster
// than llama.cpp", paragraph on the w4gemv.py kernel: each 4-bit value becomes
// the exact float (value - 8) before it is multiplied).  Every product the
// kernels form is exactly (c - 8) * x (times a power of two), so a code of 8
// contributes an exact zero and the fp32 accumulators only ever see terms of
// the size of (c - 8) * x.  Two decodes, both exact:
//
//  - fp16 (batch-1 GEMV, HBM-bound, where ALU work per code must stay small):
//    the device layout puts the codes of elements 2j and 2j+1 of an
//    8-element word at bits [4j, 4j+4) and [16+4j, 20+4j).  Masking nibble 0
//    (or 1) of both halves into the mantissa of the fp16 pair (1024, 1024)
//    gives the exact fp16 pair (1024 + c, ...) (or (1024 + 16c, ...)), and one
//    packed fp16 add (or multiply-add by 1/16) turns it into (c - 8, ...),
//    exactly: every intermediate is an integer (or a sixteenth) inside fp16's
//    exact range.  The activation elements a lane holds (its 32-element
//    chunks) are scaled by one power of two 2^s and rounded to fp16, which is
//    exact whenever every nonzero one is a normal bf16 within 2^29 of the
//    largest of them; v_dot2_f32_f16 then forms exact products.  A lane whose
//    elements fall outside that range (or hold inf / NaN) sends its wave to
//    the bf16 decode.
//  - bf16 (matrix cores, small M, and the fallback): the nibble is moved to
//    the top of a byte and its offset bit flipped, so the byte read as a
//    signed integer is 16 (c - 8); one byte-select convert per code and one
//    pack per pair give the exact bf16 pair (16 (c_2j - 8), 16 (c_2j+1 - 8)),
//    the activations stay bf16, and the scale carries the factor 1/16.
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
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
    return __uint_as_float(h << 16);
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;  // NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// bf16 pair dot product into fp32: a.lo * b.lo + a.hi * b.hi + c.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c,
                                           false);
}

// fp16 pair dot product into fp32.
__device__ __forceinline__ float dot2h(f16x2 a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(a, __builtin_bit_cast(f16x2, b), c, false);
}

// ------------------------------------------------------ fp16 exact decode --
// The decode constants as opaque VGPR values: with the masks and the magic
// in registers the compiler selects one v_and_or_b32 per operand pair (gfx9
// VOP3 encodings take no literal constants).
struct DecodeConsts {
    uint32_t m0, m1, magic;   // masks of nibbles 0 and 1 of both halves; fp16 (1024, 1024)
    f16x2 add0;               // (-1032, -1032)
    f16x2 mul1, add1;         // (1/16, 1/16), (-72, -72)
};
__device__ __forceinline__ DecodeConsts decode_consts() {
    DecodeConsts k;
    asm volatile("v_mov_b32 %0, 0xf000f" : "=v"(k.m0));
    asm volatile("v_mov_b32 %0, 0xf000f0" : "=v"(k.m1));
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(k.magic));
    k.add0 = f16x2{(_Float16)-1032.0f, (_Float16)-1032.0f};
    k.mul1 = f16x2{(_Float16)0.0625f, (_Float16)0.0625f};
    k.add1 = f16x2{(_Float16)-72.0f, (_Float16)-72.0f};
    return k;
}

// Pair (c_2j - 8, c_2j+1 - 8) of device word w for j = 0 (nibble 0 of each
// half) and j = 1 (nibble 1); pairs 2 and 3 are pairs 0 and 1 of w >> 8.
__device__ __forceinline__ f16x2 dec16_n0(uint32_t w, const DecodeConsts& k) {
    return __builtin_bit_cast(f16x2, (w & k.m0) | k.magic) + k.add0;      // (1024 + c) - 1032
}
__device__ __forceinline__ f16x2 dec16_n1(uint32_t w, const DecodeConsts& k) {
    return __builtin_bit_cast(f16x2, (w & k.m1) | k.magic) * k.mul1 + k.add1;  // (64 + c) - 72
}

// One 32-element chunk: sum of (c_k - 8) * xh_k, with q the chunk's 4 device
// words and xh its 16 fp16 activation pairs (pair i = elements 2i, 2i+1, in
// the chunk's scaled units).  Products are exact; two fp32 chains.
__device__ __forceinline__ float chunk_dot16(u32x4 q, const uint32_t* xh, const DecodeConsts& k) {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t w = q[d];
        const uint32_t v = w >> 8;
        a0 = dot2h(dec16_n0(w, k), xh[4 * d + 0], a0);
        a1 = dot2h(dec16_n1(w, k), xh[4 * d + 1], a1);
        a0 = dot2h(dec16_n0(v, k), xh[4 * d + 2], a0);
        a1 = dot2h(dec16_n1(v, k), xh[4 * d + 3], a1);
    }
    return a0 + a1;
}

// Magnitude range of n bf16 activation pairs: the largest magnitude bits
// (mx) and the smallest nonzero magnitude bits minus one (mn; 0xFFFF when
// every element is zero), per half.
__device__ __forceinline__ void pairs_range(const uint32_t* xr, int n, u16x2& mx, u16x2& mn) {
    const u16x2 one = {1, 1};
#pragma unroll
    for (int i = 0; i < n; ++i) {
        const u16x2 mag = __builtin_bit_cast(u16x2, xr[i] & 0x7FFF7FFFu);
        mx = __builtin_elementwise_max(mx, mag);
        mn = __builtin_elementwise_min(mn, (u16x2)(mag - one));   // zero wraps to 0xFFFF
    }
}

// The power-of-two scale exponent s for a range (pairs_range over every
// element that shares it): s = min(142 - e_max, 126), e_max the largest
// biased bf16 exponent present, puts the largest magnitude below 2^16
// (fp16's largest finite value is 65504 >= 255 * 2^8) and keeps 2^-s a
// normal fp32.  `ok` is cleared unless the conversion is exact: every
// nonzero element normal (biased exponent >= 1) and within 2^29 of the
// largest (so it lands on a normal fp16), and no inf or NaN.
__device__ __forceinline__ int f16_scale_exp(u16x2 mx, u16x2 mn, bool& ok) {
    const uint32_t big = mx[0] > mx[1] ? mx[0] : mx[1];
    const uint32_t low = (mn[0] < mn[1] ? mn[0] : mn[1]) + 1u;   // 0x10000: all zero
    const int emax = (int)(big >> 7);
    const int emin = (int)(low >> 7);
    if (emax >= 255 || (low < 0x10000u && (emin < 1 || emin < emax - 29))) ok = false;
    return 142 - emax < 126 ? 142 - emax : 126;
}

// n bf16 activation pairs -> fp16 pairs of x * 2^s, in place.
__device__ __forceinline__ void pairs_to_f16(uint32_t* xr, int n, int s) {
#pragma unroll
    for (int i = 0; i < n; ++i) {
        const f32x2 f = {ldexpf(__uint_as_float(xr[i] << 16), s),
                         ldexpf(__uint_as_float(xr[i] & 0xFFFF0000u), s)};
        xr[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
    }
}

// Converts NC chunks of bf16 activation pairs (16 pairs each) in place to
// fp16 pairs of x * 2^s with one shared scale (f16_scale_exp) and returns
// 2^-s.
template <int NC>
__device__ __forceinline__ float chunks_to_f16(uint32_t (&xr)[NC][16], bool& ok) {
    u16x2 mx = {0, 0}, mn = {0xFFFF, 0xFFFF};
#pragma unroll
    for (int c = 0; c < NC; ++c) pairs_range(xr[c], 16, mx, mn);
    const int s = f16_scale_exp(mx, mn, ok);
#pragma unroll
    for (int c = 0; c < NC; ++c) pairs_to_f16(xr[c], 16, s);
    return ldexpf(1.0f, -s);
}

__device__ __forceinline__ float chunk_to_f16(uint32_t (&xr)[16], bool& ok) {
    return chunks_to_f16<1>(reinterpret_cast<uint32_t (&)[1][16]>(xr), ok);
}

// ------------------------------------------------------ bf16 exact decode --
// Device word w -> the bf16 pairs (16 (c_2j - 8), 16 (c_2j+1 - 8)),
// j = 0..3, in element order.  Byte b of w holds nibble positions 2b and
// 2b + 1, i.e. elements (0, 2), (4, 6), (1, 3), (5, 7) for b = 0..3.
__device__ __forceinline__ float sbyte16(uint32_t v, int b) {
    return (float)(int)(int8_t)(v >> (8 * b));
}
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    const f32x2 f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}
__device__ __forceinline__ u32x4 decode_x16(uint32_t w) {
    const uint32_t hi = (w & 0xF0F0F0F0u) ^ 0x80808080u;          // elements 2, 6, 3, 7
    const uint32_t lo = ((w << 4) & 0xF0F0F0F0u) ^ 0x80808080u;   // elements 0, 4, 1, 5
    return u32x4{pack_bf16(sbyte16(lo, 0), sbyte16(lo, 2)), pack_bf16(sbyte16(hi, 0), sbyte16(hi, 2)),
                 pack_bf16(sbyte16(lo, 1), sbyte16(lo, 3)), pack_bf16(sbyte16(hi, 1), sbyte16(hi, 3))};
}

// One 32-element chunk: sum of 16 (c_k - 8) * x_k with bf16 activation pairs
// xr (exact products; two fp32 chains).  The caller scales by s / 16.
__device__ __forceinline__ float chunk_dot_x16(u32x4 q, const uint32_t* xr) {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const u32x4 b = decode_x16(q[d]);
        a0 = dot2(b[0], xr[4 * d + 0], a0);
        a1 = dot2(b[1], xr[4 * d + 1], a1);
        a0 = dot2(b[2], xr[4 * d + 2], a0);
        a1 = dot2(b[3], xr[4 * d + 3], a1);
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

// Agent-scope store of an output: visible to every CU once it completes.
__device__ __forceinline__ void store_out_agent(void* y, size_t i, float v, int ydt) {
    if (ydt == W4_BF16)
        __hip_atomic_store(static_cast<uint16_t*>(y) + i, (uint16_t)f32_to_bf16_rne(v),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        __hip_atomic_store(static_cast<uint32_t*>(y) + i, __float_as_uint(v), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_out(void* y, size_t i, float v, int ydt) {
    if (ydt == W4_BF16)
        gstore(static_cast<uint16_t*>(y) + i, (uint16_t)f32_to_bf16_rne(v));
    else
        gstore(static_cast<float*>(y) + i, v);
}

}  // namespace w4
