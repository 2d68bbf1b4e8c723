// w4_persist.hip -- the independent-op persistent kernel (W4_SWEEP_STREAM);
// the decode-ordered one is in w4_ordered.hip.
//
// [P1] "Gemma 4 E2B on a 4 GB GPU with plain PyTorch, faster than llama.cpp":
// a decode step is hundreds of small kernels and launching them costs more
// than running them (paragraph on the captured graph); the speed limit is how
// fast the weights are read (paragraph on the w4gemv.py kernel).  On MI355X a
// config-sized GEMV moves 2-11 MB, which the HBM streams in about 0.3-1.3 us,
// so kernel boundaries (launch, ramp-up, drain) cost as much as the work.
// STREAM mode runs all ops of a step as one kernel with no op-to-op ordering
// (see stream_kernel): the upper bound of the step's weight streaming.
#include "w4_gemv_core.h"
#include "w4_persist.h"

namespace w4 {

#ifndef W4_STREAM_STAGES
#define W4_STREAM_STAGES 2
#endif
// Two waves per SIMD (8 per CU, 256 VGPRs each, no spills): measured
// 150.4-151.2 us per graph-replayed step against 153.8-154.0 with four
// (128 VGPRs, 34 spilled outside the loops); three stages per wave 152-158.
#ifndef W4_STREAM_WAVES_PER_EU
#define W4_STREAM_WAVES_PER_EU 2
#endif
constexpr int kStreamStages = W4_STREAM_STAGES;  // register stages per wave

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
        gemv_rows_generic<L>(a, rg0, rg1, 1, lane);
}

// (register budget for W4_STREAM_WAVES_PER_EU waves per SIMD: 2 -> 256 VGPRs)
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

// Occupancy of the persistent kernels.  The decode-ordered kernel's LDS
// (above 64 KB) needs its limit raised, once per device (setting it again is
// harmless).
int persist_occupancy(bool dep, int* blocks_per_cu) {
    if (!dep)
        return hip_fail(hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, stream_kernel,
                                                                     kPwThreads, 0),
                        "occupancy");
    int st = hip_fail(hipFuncSetAttribute(reinterpret_cast<const void*>(&ordered_kernel),
                                          hipFuncAttributeMaxDynamicSharedMemorySize,
                                          ordered_lds_bytes()),
                      "ordered kernel LDS limit");
    if (st != W4_OK) return st;
    return hip_fail(hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, ordered_kernel,
                                                                 kOrdThreads,
                                                                 ordered_lds_bytes()),
                    "occupancy");
}

int launch_persist(bool dep, const SweepOp* ops_dev, int n_ops, SweepCtl* ctl,
                   const int* range, int grid, int first0, int first1, int pre,
                   unsigned poll_limit, hipStream_t s) {
    if (dep)
        ordered_kernel<<<dim3(grid), dim3(kOrdThreads), ordered_lds_bytes(), s>>>(
            ops_dev, n_ops, ctl, first0, first1, pre, poll_limit);
    else
        stream_kernel<<<dim3(grid), dim3(kPwThreads), 0, s>>>(ops_dev, n_ops, range);
    return hip_fail(hipGetLastError(), "persistent sweep launch");
}

}  // namespace w4
