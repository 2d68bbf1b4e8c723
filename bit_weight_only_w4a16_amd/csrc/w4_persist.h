// w4_persist.h -- device-side op table and control block of the persistent
// decode-step kernel (internal).
#pragma once

#include "w4_dispatch.h"

namespace w4 {

constexpr int kPwWaves = 4;                 // waves per workgroup
constexpr int kPwThreads = 64 * kPwWaves;
constexpr int kPwMaxU = 4;                  // chunks per lane per row
constexpr int kPwMaxC = 256;                // chunks per row (K <= 8192)

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
};

// Tile shapes (L lanes per row, U chunks per lane, L * U == C) compiled into
// the STREAM kernel; any other K runs a generic loop.
// At most 3 chunks per lane keeps the kernel at <= 128 VGPRs (4 waves per
// SIMD); shapes are tried in order, so K = 2048 takes 32 x 2.
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

// Control block: launch counter (epochs), error word, one flag per workgroup.
struct SweepCtl {
    unsigned launch_count;
    unsigned error;
    unsigned pad[62];
    unsigned flags[1];
};

inline size_t sweep_ctl_bytes(int grid) {
    return sizeof(SweepCtl) + sizeof(unsigned) * (size_t)grid;
}

int persist_occupancy(bool dep, int* blocks_per_cu);
int launch_persist(bool dep, const SweepOp* ops_dev, int n_ops, SweepCtl* ctl,
                   const int* range, int grid, hipStream_t s);

}  // namespace w4
