// w4_aux.hip -- the packer and the memory probes.
//
// Packer: [P2] "fastgemma -- Gemma 4 E2B, CPU-only, AMX INT8 / AVX-512 VNNI",
// section "What is in the file": weights are packed once into the order the
// kernel loads them, so nothing is repacked at run time.  Here that order is
// the canonical row-major code layout with each word's nibbles regrouped
// (even elements in the low half-word, odd in the high) so one and-or per
// element pair yields a bf16 operand pair; scales follow at a 256-byte
// boundary.
//
// Probes: [P1] "Gemma 4 E2B on a 4 GB GPU with plain PyTorch, faster than
// llama.cpp", the summary line of the w4gemv.py kernel compares the kernel
// with a plain sum over memory; the copy kernel calibrates byte counters; the
// handoff probe measures the fixed cost of one op of a decode step whose ops
// each read the whole previous output (the paragraph on the decode step
// captured once as a graph).
#include "w4_dispatch.h"
#include "w4_ring.h"

namespace w4 {

__global__ __launch_bounds__(256) void pack_kernel(const uint32_t* __restrict__ P,
                                                   const uint16_t* __restrict__ S,
                                                   uint32_t* __restrict__ codes,
                                                   uint16_t* __restrict__ scales,
                                                   size_t n_words, size_t n_scales) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += stride)
        codes[i] = word_to_device(P[i]);
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_scales; i += stride)
        scales[i] = S[i];
}

int launch_pack(const uint32_t* P, const uint16_t* S, int N, int K, int group,
                void* out, hipStream_t s) {
    const size_t n_words = (size_t)N * (size_t)(K / 8);
    const size_t n_scales = (size_t)N * (size_t)(K / group);
    uint8_t* base = static_cast<uint8_t*>(out);
    size_t blocks = (n_words + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    pack_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
        P, S, reinterpret_cast<uint32_t*>(base),
        reinterpret_cast<uint16_t*>(base + scale_offset(N, K)), n_words, n_scales);
    return hip_fail(hipGetLastError(), "pack launch");
}

__global__ void zero_u32_kernel(uint32_t* p) {
    if (threadIdx.x == 0 && blockIdx.x == 0) p[0] = 0u;
}

// Each wave sums its own contiguous slice of the buffer, 1 KB per load
// instruction, 8 non-temporal loads in flight per lane (the access pattern
// that reads fastest on gfx950); the remainder is summed grid-stride.
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ buf,
                                                         size_t n16, uint32_t* out) {
    constexpr int kUnroll = 8;
    const int lane = threadIdx.x & 63;
    const size_t nw = (size_t)gridDim.x * (blockDim.x >> 6);
    const size_t gw = (size_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const size_t per = n16 / nw / (64 * kUnroll) * (64 * kUnroll);  // per wave
    uint32_t acc = 0u;
    const u32x4* p = buf + gw * per + lane;
    for (size_t j = 0; j < per; j += 64 * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = nt_load(p + j + 64 * u);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc += v[u][0] + v[u][1] + v[u][2] + v[u][3];
    }
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = per * nw + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
         i += stride) {
        const u32x4 a = nt_load(buf + i);
        acc += a[0] + a[1] + a[2] + a[3];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) atomicAdd(out, acc);
}

int launch_probe_read(const void* buf, size_t bytes, uint32_t* out, hipStream_t s) {
    zero_u32_kernel<<<1, 64, 0, s>>>(out);
    const size_t n16 = bytes / 16;
    // up to 2048 waves (8 per CU); fewer for small buffers
    size_t blocks = (n16 + 256 * 8 - 1) / (256 * 8);
    const size_t cap = (size_t)kNumCUs * 2;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    probe_read_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
        static_cast<const u32x4*>(buf), n16, out);
    return hip_fail(hipGetLastError(), "probe read launch");
}

__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4* __restrict__ src,
                                                         u32x4* __restrict__ dst,
                                                         size_t n16) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        __builtin_nontemporal_store(nt_load(src + i), dst + i);
}

// Matrix-core throughput: every wave runs `iters` rounds of 16 independent
// v_mfma_f32_16x16x32_bf16 chains (no memory traffic), two waves per SIMD as
// the prefill kernels run.  The sum of the accumulators is stored only if it
// is negative, which it never is (all operands are positive), so the work
// cannot be dropped and nothing is written.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void probe_mfma_kernel(int iters, float* out) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const uint32_t lane = threadIdx.x & 63;
    // bf16 pairs of values in [1, 2): 0x3F80 | small mantissa bits
    const u32x4 a = {0x3F803F80u | (lane & 7u), 0x3F813F80u, 0x3F823F80u, 0x3F833F80u | (lane >> 3)};
    const u32x4 b = {0x3F843F80u, 0x3F853F80u | (lane & 3u), 0x3F863F80u, 0x3F873F80u};
    f32x4 acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                             __builtin_bit_cast(bf16x8, b),
                                                             acc[j], 0, 0, 0);
    }
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) sum += (acc[j][0] + acc[j][1]) + (acc[j][2] + acc[j][3]);
    if (sum < 0.f) gstore(out, sum);
}

int launch_probe_mfma(int iters, float* out, hipStream_t s) {
    probe_mfma_kernel<<<dim3(kNumCUs * 2), dim3(256), 0, s>>>(iters, out);
    return hip_fail(hipGetLastError(), "probe mfma launch");
}

int launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
    const size_t n16 = bytes / 16;
    size_t blocks = (n16 + 255) / 256;
    const size_t cap = (size_t)kNumCUs * 8;
    if (blocks > cap) blocks = cap;
    probe_copy_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
        static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
    return hip_fail(hipGetLastError(), "probe copy launch");
}

// Grid-wide handoff probe: the per-op handoff of the decode-ordered sweep
// kernel with no weights, so that its cost is measured apart from any GEMV.
// One workgroup of one wave per CU.  Round r: every workgroup stores `rows`
// bf16 values (its share of a vector of G * rows elements, buffer r mod 2) at
// agent scope, waits for them to complete and adds one to its XCD's counter
// (workgroup w counts in counter w mod 8, each counter in its own 128-byte
// line); lanes 0..7 then poll the eight counters (lane 8 the error word) until
// they sum to (r + 1) G, and the wave loads the whole vector into LDS with
// agent-scope 16-byte global-to-LDS loads and waits for them, as the sweep
// kernel's control wave does before every op.  rows = 0 is the bare
// signal-and-poll round.  A poll that gives up sets the error word and every
// workgroup leaves.
namespace {
constexpr int kHoCtlWords = 512;                       // error word, 8 counters
constexpr int kHoMaxRows = 64;
constexpr size_t kHoVecBytes = (size_t)kNumCUs * kHoMaxRows * 2;
constexpr unsigned kHoPollLimit = 1u << 20;

__device__ __forceinline__ void dma16_agent_probe(uint32_t off, const void* base, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 sc1"
                 :
                 : "v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
}
}  // namespace

__global__ __launch_bounds__(64) void probe_handoff_kernel(unsigned* ctl, uint16_t* y0,
                                                           uint16_t* y1, int rounds, int rows) {
    __shared__ __align__(16) uint8_t xs[kHoVecBytes];
    const int lane = threadIdx.x;
    const int w = blockIdx.x;
    const unsigned G = gridDim.x;
    // 16-byte pieces of the vector; lanes past the last re-read it into the
    // part of xs past the vector (xs holds kHoVecBytes / 16 pieces, a
    // multiple of 64 at or above every piece count)
    const int n16 = ((int)G * rows * 2 + 15) / 16;
    const unsigned* p = lane < 8 ? &ctl[32 + 32 * lane] : &ctl[0];
    for (int r = 0; r < rounds; ++r) {
        uint16_t* y = (r & 1) ? y1 : y0;
        if (lane < rows)
            __hip_atomic_store(y + (size_t)w * rows + lane, (uint16_t)(r + lane),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);   // the stores are visible to every CU
        asm volatile("" ::: "memory");
        if (lane == 0)
            __hip_atomic_fetch_add(&ctl[32 + 32 * (w & 7)], 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        const unsigned target = (unsigned)(r + 1) * G;
        bool ok = false;
        for (unsigned spin = 0; spin < kHoPollLimit; ++spin) {
            const unsigned v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            unsigned c = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) c += __builtin_amdgcn_readlane(v, j);
            const unsigned e = __builtin_amdgcn_readlane(v, 8);
            if ((int)(c - target) >= 0) {
                ok = true;
                break;
            }
            if (e) break;
        }
        if (!ok) {
            if (lane == 0) __hip_atomic_store(&ctl[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        for (int j = 0; j < n16; j += 64) {
            const int q = j + lane < n16 ? j + lane : n16 - 1;
            dma16_agent_probe(16u * (uint32_t)q, y, ring::lds_addr(xs + 16 * j));
        }
        ring::wait_vm<0>();
    }
}

size_t probe_handoff_bytes() { return (size_t)kHoCtlWords * 4 + 2 * kHoVecBytes; }

int launch_probe_handoff(void* work, int rounds, int rows, hipStream_t s) {
    uint8_t* base = static_cast<uint8_t*>(work);
    unsigned* ctl = reinterpret_cast<unsigned*>(base);
    uint16_t* y0 = reinterpret_cast<uint16_t*>(base + kHoCtlWords * 4);
    uint16_t* y1 = reinterpret_cast<uint16_t*>(base + kHoCtlWords * 4 + kHoVecBytes);
    int st = hip_fail(hipMemsetAsync(ctl, 0, kHoCtlWords * 4, s), "probe handoff clear");
    if (st != W4_OK) return st;
    probe_handoff_kernel<<<dim3(kNumCUs), dim3(64), 0, s>>>(ctl, y0, y1, rounds, rows);
    return hip_fail(hipGetLastError(), "probe handoff launch");
}

}  // namespace w4
