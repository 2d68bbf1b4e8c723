// w4_persist.hip -- one persistent kernel that walks a decode step's GEMVs.
//
// [P1] "Gemma 4 E2B on a 4 GB GPU with plain PyTorch, faster than llama.cpp":
// a decode step is hundreds of small kernels and launching them costs more
// than running them (paragraph on the captured graph); the speed limit is how
// fast the weights are read (paragraph on the w4gemv.py kernel).  On MI355X a
// config-sized GEMV moves 2-11 MB, which the HBM streams in about 0.3-1.3 us,
// so kernel boundaries (launch, ramp-up, drain) cost as much as the work.
// Two persistent kernels replace the per-GEMV launches.  STREAM mode (ops
// independent) is described at stream_kernel.  PERSISTENT mode keeps decode
// order:
//
//  - Tiles.  A tile is one row group of one op (64/L rows; L lanes per row,
//    lane l owning chunks l, l + L, ...).  Wave g of the grid takes row groups
//    g, g + GW, ... of every op, rotated per op so the ops' tails spread over
//    different waves.
//  - Weight prefetch.  Each wave keeps the codes and scales of its next tile in
//    registers while it computes the current one; the next tile may belong to
//    a later op, so weight streaming crosses op boundaries (weights never
//    depend on activations).
//  - Activations.  Each workgroup stages op i's activation vector and its
//    per-chunk offset terms in one of two LDS slots; waves read their chunk
//    slices from LDS.
//  - Ordering (PERSISTENT mode).  Before a workgroup reads op i's activations
//    it waits until every workgroup has published "op i-1 done" (one flag
//    word per workgroup); so nothing of op i is computed before op i-1's
//    outputs are all written, as in a decode step.  Outputs are stored and
//    activations loaded with agent-scope (L2-bypassing) accesses, and a
//    workgroup publishes its flag only after its output stores have
//    completed, so no whole-L2 write-back or invalidate is needed (those
//    cost ~11 us per op: 2.5 ms against 0.93 ms per sweep).
//  - Safety.  Flags carry an epoch (launch count / grid) so replays need no
//    reset.  Every wait is bounded; a wait that gives up sets an error word,
//    and every other wait then gives up too, so the grid always drains.
#include "w4_gemv_core.h"
#include "w4_persist.h"

namespace w4 {

constexpr unsigned kSpinLimit = 1u << 18;
#ifndef W4_STREAM_STAGES
#define W4_STREAM_STAGES 2
#endif
#ifndef W4_STREAM_WAVES_PER_EU
#define W4_STREAM_WAVES_PER_EU 4
#endif
constexpr int kStreamStages = W4_STREAM_STAGES;  // register stages per wave

struct TileRegs {
    u32x4 q[kPwMaxU];
    uint32_t s[kPwMaxU];
};

__device__ __forceinline__ int first_rg(const SweepOp& op, int gw, int GW) {
    int r = (gw - op.rot) % GW;
    return r < 0 ? r + GW : r;
}

// Moves (i, rg) to the first tile at or after it that exists.
__device__ __forceinline__ void settle(const SweepOp* ops, int n_ops, int gw, int GW, int& i,
                                       int& rg) {
    while (i < n_ops && rg >= ops[i].NG) {
        ++i;
        if (i < n_ops) rg = first_rg(ops[i], gw, GW);
    }
}

__device__ __forceinline__ void load_tile(const SweepOp& op, int rg, int lane, TileRegs& t) {
    const int lk = lane & (op.L - 1);
    const int lr = lane >> op.lshift;
    int n = rg * op.R + lr;
    n = n < op.N ? n : op.N - 1;
    const u32x4* cp = op.codes + (size_t)n * op.C;
    const uint16_t* sp = op.scales + (size_t)n * op.G;
#pragma unroll
    for (int u = 0; u < kPwMaxU; ++u) {
        if (u < op.U) {
            int c = lk + op.L * u;
            c = c < op.C ? c : op.C - 1;
            t.q[u] = nt_load(cp + c);
            t.s[u] = gload(sp + (c >> op.gshift));
        }
    }
}

// Agent-scope stores of an output: visible to every CU once they complete.
__device__ __forceinline__ void store_out_agent(void* y, size_t i, float v, int ydt) {
    if (ydt == W4_BF16)
        __hip_atomic_store(static_cast<uint16_t*>(y) + i, (uint16_t)f32_to_bf16_rne(v),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        __hip_atomic_store(static_cast<uint32_t*>(y) + i, __float_as_uint(v), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void compute_tile(const SweepOp& op, int rg, int lane,
                                             const TileRegs& t, const uint32_t* xs,
                                             const float* bs, const DecodeConsts& k) {
    const int lk = lane & (op.L - 1);
    const int lr = lane >> op.lshift;
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < kPwMaxU; ++u) {
        if (u < op.U) {
            const int c = lk + op.L * u;
            if (c < op.C) {
                uint32_t xr[16];
                const u32x4* p = reinterpret_cast<const u32x4*>(xs + 16 * c);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const u32x4 v = p[i];
                    xr[4 * i + 0] = v[0];
                    xr[4 * i + 1] = v[1];
                    xr[4 * i + 2] = v[2];
                    xr[4 * i + 3] = v[3];
                }
                acc = fmaf(bf16_to_f32(t.s[u]), chunk_dot(t.q[u], xr, k) + bs[c], acc);
            }
        }
    }
    if (op.L == 16)
        acc = group_sum<16>(acc);
    else if (op.L == 32)
        acc = group_sum<32>(acc);
    else
        acc = group_sum<64>(acc);
    const int n = rg * op.R + lr;
    if (lk == 0 && n < op.N) store_out_agent(op.y, (size_t)n, acc, op.ydt);
}

// Thread t < C writes chunk t of the activation (held in v) and its negated
// offset term into the LDS slot.
__device__ __forceinline__ void put_chunk(const u32x4 (&v)[4], int t, uint32_t* xs, float* bs) {
    uint32_t xr[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        reinterpret_cast<u32x4*>(xs + 16 * t)[i] = v[i];
        xr[4 * i + 0] = v[i][0];
        xr[4 * i + 1] = v[i][1];
        xr[4 * i + 2] = v[i][2];
        xr[4 * i + 3] = v[i][3];
    }
    bs[t] = -chunk_bias(xr);
}

// Agent-scope loads of an activation chunk (an activation written by another
// CU's op is never read from a stale L2 line).
__device__ __forceinline__ void get_chunk(const SweepOp& op, int t, u32x4 (&v)[4]) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(op.x + 4 * t);
#pragma unroll
    for (int i = 0; i < 16; ++i)
        v[i >> 2][i & 3] = __hip_atomic_load(p + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned wave_min(unsigned v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const unsigned o = __shfl_xor(v, off, 64);
        v = o < v ? o : v;
    }
    return v;
}

// Wave 0 polls every workgroup's flag until all reached `target` (wrap-safe),
// the error word is set, or the spin limit passes.  Returns, to every thread
// of the workgroup, whether the wait succeeded.
__device__ __forceinline__ bool wait_all(SweepCtl* ctl, int nflags, unsigned target, int wave,
                                         int lane, int* s_ok) {
    if (wave == 0) {
        bool ok = false;
        for (unsigned spin = 0; spin < kSpinLimit; ++spin) {
            unsigned mn = 0xFFFFFFFFu;
            for (int j = lane; j < nflags; j += 64) {
                const unsigned f = __hip_atomic_load(&ctl->flags[j], __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                const unsigned d = f - target;  // >= 0 (as signed) once reached
                const unsigned reached = (int)d >= 0 ? 1u : 0u;
                mn = reached < mn ? reached : mn;
            }
            mn = wave_min(mn);
            if (mn == 1u) {
                ok = true;
                break;
            }
            const unsigned err =
                __hip_atomic_load(&ctl->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (err != 0u) break;
            __builtin_amdgcn_s_sleep(1);
        }
        if (lane == 0) {
            if (!ok)
                __hip_atomic_store(&ctl->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *s_ok = ok ? 1 : 0;
        }
    }
    __syncthreads();
    return *s_ok != 0;
}

// PERSISTENT mode: decode order.  Every workgroup takes part in every op
// (tile rotation over all waves) and waits for op i-1 before reading op i's
// activations.
__global__ __launch_bounds__(kPwThreads) void ordered_kernel(const SweepOp* __restrict__ ops,
                                                             int n_ops, SweepCtl* ctl) {
    __shared__ __align__(16) uint32_t xs[2][kPwMaxC * 16];
    __shared__ float bs[2][kPwMaxC];
    __shared__ unsigned s_epoch;
    __shared__ int s_ok;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int GW = gridDim.x * kPwWaves;
    const int gw = blockIdx.x * kPwWaves + wave;
    const DecodeConsts k = decode_consts();

    if (tid == 0) s_epoch = atomicAdd(&ctl->launch_count, 1u) / gridDim.x;
    __syncthreads();
    const unsigned ebase = s_epoch * (unsigned)n_ops;

    // this wave's tile cursor and its prefetched registers
    int pi = 0, prg = first_rg(ops[0], gw, GW);
    settle(ops, n_ops, gw, GW, pi, prg);
    TileRegs cur, nxt;
    if (pi < n_ops) load_tile(ops[pi], prg, lane, cur);

    u32x4 xv[4];

    for (int i = 0; i < n_ops; ++i) {
        const SweepOp op = ops[i];
        const int slot = i & 1;
        if (i > 0 && !wait_all(ctl, gridDim.x, ebase + (unsigned)i, wave, lane, &s_ok))
            return;
        if (tid < op.C) {
            get_chunk(op, tid, xv);
            put_chunk(xv, tid, xs[slot], bs[slot]);
        }
        __syncthreads();

        while (pi == i) {
            int ni = pi, nrg = prg + GW;
            settle(ops, n_ops, gw, GW, ni, nrg);
            if (ni < n_ops) load_tile(ops[ni], nrg, lane, nxt);
            compute_tile(op, prg, lane, cur, xs[slot], bs[slot], k);
            cur = nxt;
            pi = ni;
            prg = nrg;
        }

        // publish "op i done": every wave waits until its agent-scope output
        // stores have completed (all counters 0: the stores may be flat
        // accesses, which count in vmcnt and lgkmcnt), the barrier joins the
        // waves, then the flag
        __builtin_amdgcn_s_waitcnt(0);
        asm volatile("" ::: "memory");
        __syncthreads();
        if (tid == 0)
            __hip_atomic_store(&ctl->flags[blockIdx.x], ebase + (unsigned)i + 1u,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// STREAM mode: independent ops.  The concatenated tile list of all ops is cut
// into one contiguous, byte-balanced range per wave (range[w] .. range[w+1];
// range[waves + 1 + w] is the op that holds tile range[w]),
// so each wave streams about total/waves bytes, crossing only the few op
// boundaries inside its range.  Within one op the wave runs the batch-1 GEMV
// inner loop over consecutive row groups (activation slice in registers, next
// row group in flight); there is no LDS, no barrier and no communication
// between waves.  The op's tile shape (L, U) selects a compiled loop.
// (Handing tiles out through a per-workgroup counter evens out the waves'
// finishing times but measured slower: the counter sits between one tile's
// compute and the next tile's loads.)
template <int L, int U>
__device__ __forceinline__ void stream_rows(const SweepOp& op, int rg0, int rg1, int lane,
                                            const DecodeConsts& k) {
    GemvArgs a;
    a.codes = op.codes;
    a.scales = op.scales;
    a.x = reinterpret_cast<const uint32_t*>(op.x);
    a.y = op.y;
    a.N = op.N;
    a.C = op.C;
    a.G = op.G;
    a.gshift = op.gshift;
    a.ydt = op.ydt;
    if (U > 0)
        gemv_rows<L, (U > 0 ? U : 1), true, kStreamStages, true>(a, rg0, rg1, 1, lane, k);
    else
        gemv_rows_generic<L>(a, rg0, rg1, 1, lane, k);
}

// (register budget for W4_STREAM_WAVES_PER_EU waves per SIMD: 4 -> 128 VGPRs)
__global__ __launch_bounds__(kPwThreads)
__attribute__((amdgpu_waves_per_eu(W4_STREAM_WAVES_PER_EU)))
void stream_kernel(const SweepOp* __restrict__ ops, int n_ops, const int* __restrict__ range) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int gw = blockIdx.x * kPwWaves + wave;
    const int tb = range[gw];
    const int te = range[gw + 1];
    if (tb >= te) return;
    const DecodeConsts k = decode_consts();

    int i = range[gridDim.x * kPwWaves + 1 + gw];  // the op that holds tile tb
    for (int t = tb; t < te && i < n_ops; ++i) {
        const SweepOp op = ops[i];
        const int end = te < op.base + op.NG ? te : op.base + op.NG;
        const int rg0 = t - op.base, rg1 = end - op.base;
        switch (op.cfg) {
            case kCfg16x1: stream_rows<16, 1>(op, rg0, rg1, lane, k); break;
            case kCfg16x2: stream_rows<16, 2>(op, rg0, rg1, lane, k); break;
            case kCfg16x3: stream_rows<16, 3>(op, rg0, rg1, lane, k); break;
            case kCfg32x2: stream_rows<32, 2>(op, rg0, rg1, lane, k); break;
            case kCfg32x3: stream_rows<32, 3>(op, rg0, rg1, lane, k); break;
            case kCfg64x1: stream_rows<64, 1>(op, rg0, rg1, lane, k); break;
            case kCfg64x2: stream_rows<64, 2>(op, rg0, rg1, lane, k); break;
            case kCfg64x3: stream_rows<64, 3>(op, rg0, rg1, lane, k); break;
            default: stream_rows<16, 0>(op, rg0, rg1, lane, k); break;
        }
        t = end;
    }
}

int persist_occupancy(bool dep, int* blocks_per_cu) {
    hipError_t e =
        dep ? hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, ordered_kernel,
                                                           kPwThreads, 0)
            : hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, stream_kernel,
                                                           kPwThreads, 0);
    return hip_fail(e, "occupancy");
}

int launch_persist(bool dep, const SweepOp* ops_dev, int n_ops, SweepCtl* ctl,
                   const int* range, int grid, hipStream_t s) {
    if (dep)
        ordered_kernel<<<dim3(grid), dim3(kPwThreads), 0, s>>>(ops_dev, n_ops, ctl);
    else
        stream_kernel<<<dim3(grid), dim3(kPwThreads), 0, s>>>(ops_dev, n_ops, range);
    return hip_fail(hipGetLastError(), "persistent sweep launch");
}

}  // namespace w4
