// w4_ring.h -- helpers for kernels fed by an LDS ring that global-to-LDS
// DMA loads fill ahead of the stage being multiplied (internal).
//
// The DMA loads are issued with inline asm: the compiler, which otherwise
// waits for every such load before any LDS read that may alias it, then
// leaves all waits on them to the explicit ones here.  Its own vmcnt counts
// (for loads it does see) stay correct, only stricter, since loads complete
// in order.
#pragma once

#include <type_traits>
#include <utility>

#include "w4_common.h"

// the DMA asm clobbers M0, which the compiler reserves; no other M0 use lives
// across it in the ring kernels
#pragma clang diagnostic ignored "-Winline-asm"

namespace w4 {
namespace ring {

// s_waitcnt with vmcnt = N and the other counters left alone (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until at most LOADS * min(pending, P) of this wave's DMA ops are in
// flight (pending is wave-uniform; the branches are scalar).
template <int LOADS, int P>
__device__ __forceinline__ void wait_stage(int pending) {
    if constexpr (P == 0) {
        wait_vm<0>();
    } else {
        if (pending >= P)
            wait_vm<LOADS * P>();
        else
            wait_stage<LOADS, P - 1>(pending);
    }
}

// Workgroup barrier that is also a compiler barrier for memory operations;
// it does not wait for outstanding loads (the explicit waits do that).
__device__ __forceinline__ void ring_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One DMA load: each lane's 16 (or 4) bytes at base + off land in LDS at
// lds + 16 * lane (or 4 * lane); lds is wave-uniform.  Written as inline asm so
// that the compiler, which would otherwise wait for every such load before any
// LDS read that may alias it, leaves all waits on them to the explicit ones.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void dma16(uint32_t off, const void* base, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(uint32_t off, const void* base, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
}

// f(std::integral_constant<int, I>) for I = 0 .. N-1, unrolled
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace ring
}  // namespace w4
