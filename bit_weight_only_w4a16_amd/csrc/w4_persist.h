// w4_persist.h -- device-side op table and control block of the persistent
// decode-step kernel (internal).
#pragma once

#include "w4_dispatch.h"

namespace w4 {

constexpr int kPwWaves = 4;                 // waves per workgroup
constexpr int kPwThreads = 64 * kPwWaves;
constexpr int kPwMaxU = 4;                  // chunks per lane per row
constexpr int kPwMaxC = 256;                // chunks per row (K <= 8192)

// Decode-ordered kernel (w4_ordered.hip): 8 waves per workgroup; wave 0 the
// control wave, wave 7 the DMA wave (it fills the two LDS slots with the
// next resident ops' shares), waves 0..6 compute resident shares.
constexpr int kOrdWaves = 8;
constexpr int kOrdThreads = 64 * kOrdWaves;
constexpr int kOrdDmaWave = kOrdWaves - 1;
constexpr int kOrdCodeBytes = 49 * 1024;                 // codes per slot
constexpr int kOrdScaleBytes = 7 * 1024;                 // scales per slot
constexpr int kOrdMaxK = 32 * kPwMaxC;                   // 8192
constexpr int kOrdMaxRows = 512;                         // rows of a resident share
constexpr int kOrdGroups = 16 * (kOrdWaves - 1) / 4;     // 16-lane groups of waves 0..6
constexpr int kOrdMaxPartials = 1024;                    // rows x parts of a resident share
constexpr int kOrdPreChunks = 6;                         // chunks per lane decoded ahead

// One GEMV of the step, as the kernel reads it.
struct SweepOp {
    const u32x4* codes;      // N x C chunks
    const uint16_t* scales;  // N x G bf16
    const u32x4* x;          // K bf16
    void* y;
    int N, C, G, gshift, ydt;
    int L, lshift, U, R;     // lanes per row, log2 L, chunks per lane, rows per tile
    int NG;                  // tiles (row groups)
    int rot;                 // first wave of this op's tile rotation (decode order)
    int base;                // index of this op's first tile in the step's tile list
    int cfg;                 // STREAM: compiled tile shape (kCfg*), or kCfgGeneric
    // decode-ordered mode
    int res;                 // 1: every workgroup's share fits an LDS slot (DMA'd ahead)
    int slot;                // its slot (0 or 1)
    int next;                // resident op DMA'd into this op's slot after it (-1: none)
    int nres;                // the next resident op (-1: none)
    // resident (decode-ordered mode): tasks (part p, row r) of a share, p in
    // [0, P) of CP chunks each (UP = ceil(CP / 16) per lane), r in [0, Rm),
    // numbered t = p Rm + r; plan[g] = (first task << 16) | task count of
    // 16-lane group g of waves 0..6
    int P, CP, UP, Rm;
    const uint32_t* plan;
};

// Tile shapes (L lanes per row, U chunks per lane, L * U == C) compiled into
// the STREAM kernel; any other K runs a generic loop.
// At most 3 chunks per lane (the activation slice, 16 registers per chunk,
// stays in registers); shapes are tried in order, so K = 2048 takes 32 x 2.
enum {
    kCfgGeneric = 0,
    kCfg16x1, kCfg16x2, kCfg16x3,
    kCfg32x2, kCfg32x3,
    kCfg64x1, kCfg64x2, kCfg64x3
};

inline int stream_cfg(int C, int* L) {
    struct Shape { int cfg, L, U; };
    static const Shape shapes[] = {
        {kCfg16x3, 16, 3}, {kCfg16x2, 16, 2}, {kCfg16x1, 16, 1}, {kCfg32x3, 32, 3},
        {kCfg32x2, 32, 2}, {kCfg64x3, 64, 3}, {kCfg64x2, 64, 2}, {kCfg64x1, 64, 1}};
    for (const Shape& s : shapes)
        if (s.L * s.U == C) {
            *L = s.L;
            return s.cfg;
        }
    *L = 16;
    return kCfgGeneric;
}

// Control block: error word; the decode-ordered kernel's completion
// counters (one per XCD, each in its own 128-byte line) and the count of
// workgroups that finished a replay.
struct SweepCtl {
    unsigned error;
    unsigned pad0[31];
    unsigned cnt[8 * 32];
    unsigned fin;
    unsigned pad1[31];
};

inline size_t sweep_ctl_bytes(int) { return sizeof(SweepCtl); }

int persist_occupancy(bool dep, int* blocks_per_cu);
// poll_limit: the decode-ordered kernel's completion polls per op before it
// gives up (kOrdPollLimit unless a test asks for fewer)
constexpr unsigned kOrdPollLimit = 1u << 20;
int launch_persist(bool dep, const SweepOp* ops_dev, int n_ops, SweepCtl* ctl,
                   const int* range, int grid, int first0, int first1, int pre,
                   unsigned poll_limit, hipStream_t s);
int ordered_lds_bytes();
__global__ void ordered_kernel(const SweepOp* __restrict__ ops, int n_ops, SweepCtl* ctl,
                               int first0, int first1, int pre, unsigned poll_limit);

}  // namespace w4
