// w4_sweep.hip -- one decode step's GEMVs replayed as a single graph: one
// GEMV kernel per op (W4_SWEEP_GRAPH) or one persistent kernel for all ops
// (W4_SWEEP_PERSISTENT, W4_SWEEP_STREAM; see w4_persist.hip).
//
// [P1] "Gemma 4 E2B on a 4 GB GPU with plain PyTorch, faster than llama.cpp",
// paragraph on the decode step: hundreds of small kernels launched one at a
// time cost more than running them, so the step is captured once as a graph
// and replayed for every token.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <new>
#include <vector>

#include "w4_config.h"
#include "w4_persist.h"

struct w4_sweep {
    int mode = 0;
    std::vector<w4_gemv_op> ops;
    size_t weight_bytes = 0;
    int kernels = 0;
    int grid = 0;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    void* dev = nullptr;              // persistent modes: op table, ranges, control block
    w4::SweepCtl* ctl = nullptr;
    int* range = nullptr;             // STREAM: first tile of each wave (waves + 1)
    int first0 = -1, first1 = -1;     // PERSISTENT: first two resident ops
    int pre = 0;                      // PERSISTENT: resident shares decoded ahead
    unsigned poll_limit = 0;          // PERSISTENT: completion polls per op
};

namespace w4 {

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

static size_t out_bytes(const w4_gemv_op& op) {
    return (size_t)op.N * (op.y_dtype == W4_F32 ? 4 : 2);
}

static int check_op(const w4_gemv_op& op, int i) {
    if (op.group != 32 && op.group != 256 && op.group != 512)
        return fail(W4_ERR_SHAPE, "sweep op %d: group must be 32, 256 or 512", i);
    if (op.N < 1 || op.K < op.group || op.K % op.group != 0 || op.K > (1 << 20) ||
        op.N > (1 << 26))
        return fail(W4_ERR_SHAPE, "sweep op %d: bad shape N=%d K=%d", i, op.N, op.K);
    if (op.y_dtype != W4_F32 && op.y_dtype != W4_BF16)
        return fail(W4_ERR_DTYPE, "sweep op %d: bad output dtype", i);
    if (!op.packed || !op.x || !op.y) return fail(W4_ERR_ARG, "sweep op %d: NULL pointer", i);
    if (!aligned16(op.packed) || !aligned16(op.x))
        return fail(W4_ERR_ALIGN, "sweep op %d: packed and x must be 16-byte aligned", i);
    if ((reinterpret_cast<uintptr_t>(op.y) & (op.y_dtype == W4_F32 ? 3 : 1)) != 0)
        return fail(W4_ERR_ALIGN, "sweep op %d: y misaligned", i);
    return W4_OK;
}

// No op's output may share a byte with its own activation (other workgroups
// still read it while outputs are written) or with any op's weights (the
// persistent kernel reads a later op's weights ahead, and every replay reads
// them all again).
static int check_outputs_spare_inputs(const std::vector<w4_gemv_op>& ops) {
    for (size_t i = 0; i < ops.size(); ++i)
        if (ranges_overlap(ops[i].y, out_bytes(ops[i]), ops[i].x, (size_t)ops[i].K * 2))
            return fail(W4_ERR_ARG, "sweep op %d: y overlaps its own x", (int)i);
    for (size_t i = 0; i < ops.size(); ++i)
        for (size_t j = 0; j < ops.size(); ++j)
            if (ranges_overlap(ops[i].y, out_bytes(ops[i]), ops[j].packed,
                               w4_packed_bytes(ops[j].N, ops[j].K, ops[j].group)))
                return fail(W4_ERR_ARG, "sweep op %d: y overlaps the weights of op %d", (int)i,
                            (int)j);
    return W4_OK;
}

static int capture_graph_nodes(w4_sweep* h, hipStream_t cs) {
    for (const w4_gemv_op& op : h->ops) {
        const GemvTile t = pick_gemv_tile(op.N, op.K, op.group);
        const int st = launch_gemv(t, op.packed, op.N, op.K, op.group, op.x, op.y,
                                   op.y_dtype, cs);
        if (st != W4_OK) return st;
    }
    h->kernels = (int)h->ops.size();
    return W4_OK;
}

// Lanes per row for the persistent kernel: the smallest of 16, 32, 64 that
// keeps every lane within kPwMaxU chunks of a row.
static int persist_lanes(int C) {
    if (C <= 16 * kPwMaxU) return 16;
    if (C <= 32 * kPwMaxU) return 32;
    return 64;
}

// How a resident share is spread over the compute waves' 16-lane groups.
// A task is one row's sum over one part of its chunks (the row's C chunks cut
// into P parts of CP chunks, UP = ceil(CP / 16) chunks per lane), costing
// about 84 vector instructions per chunk decode and 25 for the row sum and
// its write.  Each group takes a contiguous run of tasks, numbered part by
// part, so its lanes reload their activation chunks only when the part
// changes.  Waves w and w + 4 share a SIMD (wave 7 issues the DMA, so wave 3
// has SIMD 3 to itself); a wave alone on its SIMD issues a chunk in 1.13x the
// time that two interleaved waves take per chunk (measured).  A wave runs as
// long as its busiest group.  For each P, whole rounds of four tasks (one per
// group of a wave) go one at a time to the wave that leaves the busiest SIMD
// least busy; the P with the cheapest busiest SIMD wins
// (the smallest P on ties: fewer partial sums), among those with no empty
// part, at most kPwMaxU chunks per lane and R P partials within the LDS
// buffer.
// pre: the tasks are decoded ahead into registers (kOrdPreChunks chunks per
// lane at most) by waves 1..6 only (wave 0, the control wave, polls
// meanwhile; it then has SIMD 0's second slot to itself, like wave 3).
// Fills plan[0 .. kOrdGroups) and returns false when no P fits.
static bool resident_plan(int R, int C, bool pre, SweepOp* t, uint32_t* plan) {
    constexpr int kWaves = kOrdGroups / 4;
    const int w0 = pre ? 1 : 0;   // first computing wave
    int best = 0;
    double best_cost = 0.0;
    int best_rounds[kWaves] = {};
    for (int P = 1; P <= kOrdGroups; ++P) {
        const int CP = (C + P - 1) / P;
        const int UP = (CP + 15) / 16;
        if ((P - 1) * CP >= C || UP > kPwMaxU || R * P > kOrdMaxPartials) continue;
        const int cap = pre ? kOrdPreChunks / UP : 1 << 20;   // tasks per group
        const double c = 84.0 * UP + 25.0;
        int rounds[kWaves] = {};
        // issue time of SIMD s: while both of its waves have rounds left they
        // interleave (one round each per 2 c); the longer one then runs alone
        // at 1.13 c per round
        auto simd_time = [&](int s) {
            const int a = s >= w0 ? rounds[s] : 0, b = s + 4 < kWaves ? rounds[s + 4] : 0;
            const int lo = a < b ? a : b, hi = a < b ? b : a;
            return c * (2.0 * lo + 1.13 * (hi - lo));
        };
        int left = R * P;
        for (; left > 0; left -= 4) {
            int pick = -1;
            double pick_t = 0.0;
            for (int w = w0; w < kWaves; ++w) {
                if (rounds[w] + 1 > cap) continue;
                rounds[w] += 1;
                double tt = 0.0;
                for (int s2 = 0; s2 < 4; ++s2) {
                    const double v = simd_time(s2);
                    tt = v > tt ? v : tt;
                }
                rounds[w] -= 1;
                if (pick < 0 || tt < pick_t) {
                    pick = w;
                    pick_t = tt;
                }
            }
            if (pick < 0) break;   // every wave at the cap
            rounds[pick] += 1;
        }
        if (left > 0) continue;
        double cost = 0.0;
        for (int s2 = 0; s2 < 4; ++s2) {
            const double v = simd_time(s2);
            cost = v > cost ? v : cost;
        }
        if (best == 0 || cost < best_cost) {
            best = P;
            best_cost = cost;
            for (int w = 0; w < kWaves; ++w) best_rounds[w] = rounds[w];
        }
    }
    if (best == 0) return false;
    t->P = best;
    t->CP = (C + best - 1) / best;
    t->UP = (t->CP + 15) / 16;
    t->Rm = R;
    int start = 0, left = R * best;
    for (int w = 0; w < kWaves; ++w) {
        const int n = best_rounds[w] * 4 < left ? best_rounds[w] * 4 : left;
        left -= n;
        for (int g = 0; g < 4; ++g) {
            const int k = n / 4 + (g < n % 4 ? 1 : 0);
            plan[4 * w + g] = ((uint32_t)start << 16) | (uint32_t)k;
            start += k;
        }
    }
    return true;
}

static int blocks_per_cu_override() {
    const char* e = getenv("W4_SWEEP_BLOCKS_PER_CU");
    const int v = e ? atoi(e) : 0;
    return (v >= 1 && v <= 16) ? v : 0;
}

static int setup_persistent(w4_sweep* h) {
    const bool dep = h->mode == W4_SWEEP_PERSISTENT;
    int occ = 0;
    int st = persist_occupancy(dep, &occ);
    if (st != W4_OK) return st;
    if (occ < 1) return fail(W4_ERR_UNSUPPORTED, "sweep: persistent kernel does not fit a CU");
    int bpc = dep ? 1 : blocks_per_cu_override();   // decode order: one per CU
    if (bpc == 0) bpc = 5;
    if (bpc > occ) bpc = occ;  // every workgroup must be resident at once
    int ncu = kNumCUs;
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.multiProcessorCount > 0)
            ncu = prop.multiProcessorCount;
    }
    h->grid = ncu * bpc;
    const int GW = h->grid * kPwWaves;  // waves of the decode-order kernel

    const int n = (int)h->ops.size();
    std::vector<SweepOp> tab(n);
    std::vector<uint32_t> plans((size_t)n * kOrdGroups, 0u);
    long long tiles_before = 0;
    for (int i = 0; i < n; ++i) {
        const w4_gemv_op& o = h->ops[i];
        SweepOp& t = tab[i];
        t.codes = static_cast<const u32x4*>(o.packed);
        t.scales = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(o.packed) +
                                                     scale_offset(o.N, o.K));
        t.x = static_cast<const u32x4*>(static_cast<const void*>(o.x));
        t.y = o.y;
        t.N = o.N;
        t.C = o.K / 32;
        t.G = o.K / o.group;
        t.gshift = ilog2(o.group / 32);
        t.ydt = o.y_dtype;
        t.res = 0;
        t.slot = 0;
        t.next = -1;
        t.nres = -1;
        t.P = t.CP = t.UP = t.Rm = 0;
        t.plan = nullptr;
        if (dep) {
            t.L = persist_lanes(t.C);
            t.cfg = kCfgGeneric;
            // resident: every workgroup's share of codes and scales fits an
            // LDS slot, both byte ranges are whole 16-byte units (a row of
            // codes is K / 2 bytes, a row of scales 2 K / group: K % 256 == 0
            // and K / group % 8 == 0), and the DMA offsets fit 32 bits
            const long long rows = (o.N + h->grid - 1) / h->grid;
            t.res = o.K % 256 == 0 && (o.K / o.group) % 8 == 0 &&
                    rows * (o.K / 2) <= kOrdCodeBytes &&
                    rows * (o.K / o.group) * 2 <= kOrdScaleBytes && rows <= kOrdMaxRows &&
                    (long long)o.N * (o.K / 2) < (1LL << 32);
            if (t.res && !resident_plan((int)rows, t.C, false, &t, &plans[(size_t)i * kOrdGroups]))
                t.res = 0;
        } else {
            t.cfg = stream_cfg(t.C, &t.L);
            if (t.G & 1) {  // the tiled loop reads scales in dword pairs
                t.cfg = kCfgGeneric;
                t.L = 16;  // the generic loop's lanes per row
            }
        }
        t.lshift = ilog2(t.L);
        t.U = (t.C + t.L - 1) / t.L;
        t.R = 64 / t.L;
        t.NG = (o.N + t.R - 1) / t.R;
        t.rot = (int)(tiles_before % GW);
        t.base = (int)tiles_before;
        tiles_before += t.NG;
    }
    if (tiles_before >= (1LL << 31)) return fail(W4_ERR_SHAPE, "sweep: too many tiles");
    if (dep) {
        // resident ops alternate between the two slots; resident op r_k is
        // DMA'd after r_{k-2} is computed (the first two at the start)
        std::vector<int> res;
        for (int i = 0; i < n; ++i)
            if (tab[i].res) res.push_back(i);
        for (size_t k = 0; k < res.size(); ++k) {
            tab[res[k]].slot = (int)(k & 1);
            tab[res[k]].next = k + 2 < res.size() ? res[k + 2] : -1;
            tab[res[k]].nres = k + 1 < res.size() ? res[k + 1] : -1;
        }
        h->first0 = res.size() > 0 ? res[0] : -1;
        h->first1 = res.size() > 1 ? res[1] : -1;
        // decode the resident shares ahead into registers when every one of
        // them fits (W4_FORCE_PATH ordered_inline: decode while multiplying)
        bool pre = !res.empty() && !(config()->force & kForceOrderedInline);
        std::vector<SweepOp> pt(res.size());
        std::vector<uint32_t> pp(res.size() * (size_t)kOrdGroups, 0u);
        for (size_t k = 0; k < res.size() && pre; ++k) {
            const w4_gemv_op& o = h->ops[res[k]];
            pt[k] = tab[res[k]];
            pre = resident_plan((o.N + h->grid - 1) / h->grid, tab[res[k]].C, true, &pt[k],
                                &pp[k * (size_t)kOrdGroups]);
        }
        if (pre) {
            for (size_t k = 0; k < res.size(); ++k) {
                tab[res[k]] = pt[k];
                std::copy(pp.begin() + k * kOrdGroups, pp.begin() + (k + 1) * kOrdGroups,
                          plans.begin() + (size_t)res[k] * kOrdGroups);
            }
        }
        h->pre = pre ? 1 : 0;
        {
            const long lim = config()->sweep_poll_limit;
            h->poll_limit = lim >= 0 ? (unsigned)lim : kOrdPollLimit;
        }
        {
            const auto cfg = config();
            char msg[160];
            snprintf(msg, sizeof msg,
                     "decode-ordered sweep: %d ops, %d resident, resident shares decoded %s",
                     n, (int)res.size(), pre ? "ahead" : "inline");
            log_dispatch(*cfg, msg);
        }
    }

    // STREAM partition: contiguous tile ranges, an equal share of the bytes
    // per wave (tiles of one op are equal-sized); then, for each wave, the
    // index of the op that holds its first tile.  (Shares weighted by a
    // wave's dispatch round and by XCD parity, fitted on earlier machines,
    // measured no better on later ones: 154.5 against 153.2 us, median of 15
    // trials each, so the shares are equal.)
    const int parts = GW;
    std::vector<int> range(2 * (size_t)parts + 1);
    {
        double total_bytes = 0.0;
        for (const w4_gemv_op& o : h->ops)
            total_bytes += (double)o.N * o.K / 2 + (double)o.N * (o.K / o.group) * 2;
        std::vector<double> cum((size_t)parts + 1, 0.0);
        for (int w = 0; w < parts; ++w) cum[w + 1] = cum[w] + 1.0;
        int b = 0;
        double at = 0.0;  // byte offset of the current tile
        for (int i = 0; i < n && b <= parts; ++i) {
            const w4_gemv_op& o = h->ops[i];
            const double tile = (double)tab[i].R * ((double)o.K / 2 + (double)(o.K / o.group) * 2);
            for (int t = 0; t < tab[i].NG; ++t) {
                while (b <= parts && at >= total_bytes * (cum[b] / cum[parts])) range[b++] = tab[i].base + t;
                at += tile;
            }
        }
        while (b <= parts) range[b++] = (int)tiles_before;
        range[0] = 0;
        range[parts] = (int)tiles_before;
        int i = 0;
        for (int w = 0; w < parts; ++w) {
            while (i < n && tab[i].base + tab[i].NG <= range[w]) ++i;
            range[parts + 1 + w] = i < n ? i : n - 1;
        }
    }

    const size_t tab_bytes = align_up(sizeof(SweepOp) * (size_t)n, kAlign);
    const size_t range_bytes = align_up(sizeof(int) * range.size(), kAlign);
    const size_t plan_bytes = align_up(sizeof(uint32_t) * plans.size(), kAlign);
    const size_t total = tab_bytes + range_bytes + plan_bytes + sweep_ctl_bytes(h->grid);
    st = hip_fail(hipMalloc(&h->dev, total), "sweep device buffer");
    if (st != W4_OK) {
        h->dev = nullptr;
        return W4_ERR_NOMEM;
    }
    uint8_t* base = static_cast<uint8_t*>(h->dev);
    h->range = reinterpret_cast<int*>(base + tab_bytes);
    uint32_t* plan_dev = reinterpret_cast<uint32_t*>(base + tab_bytes + range_bytes);
    h->ctl = reinterpret_cast<SweepCtl*>(base + tab_bytes + range_bytes + plan_bytes);
    for (int i = 0; i < n; ++i)
        if (tab[i].res) tab[i].plan = plan_dev + (size_t)i * kOrdGroups;
    st = hip_fail(hipMemcpy(plan_dev, plans.data(), sizeof(uint32_t) * plans.size(),
                            hipMemcpyHostToDevice), "sweep plans");
    if (st != W4_OK) return st;
    st = hip_fail(hipMemcpy(h->dev, tab.data(), sizeof(SweepOp) * (size_t)n,
                            hipMemcpyHostToDevice), "sweep op table");
    if (st != W4_OK) return st;
    st = hip_fail(hipMemcpy(h->range, range.data(), sizeof(int) * range.size(),
                            hipMemcpyHostToDevice), "sweep ranges");
    if (st != W4_OK) return st;
    st = hip_fail(hipMemset(h->ctl, 0, sweep_ctl_bytes(h->grid)), "sweep control block");
    if (st != W4_OK) return st;
    return hip_fail(hipDeviceSynchronize(), "sweep setup");
}

static void release(w4_sweep* h) {
    if (h->exec) (void)hipGraphExecDestroy(h->exec);
    if (h->graph) (void)hipGraphDestroy(h->graph);
    if (h->dev) (void)hipFree(h->dev);
    delete h;
}

}  // namespace w4

using namespace w4;

extern "C" {

int w4_decode_sweep_create(const w4_gemv_op* ops, int n_ops, int mode, void* stream,
                           w4_sweep** out) {
    (void)stream;
    if (!out) return fail(W4_ERR_ARG, "sweep: out is NULL");
    *out = nullptr;
    if (!ops || n_ops < 1) return fail(W4_ERR_ARG, "sweep: no ops");
    if (mode != W4_SWEEP_GRAPH && mode != W4_SWEEP_PERSISTENT && mode != W4_SWEEP_STREAM)
        return fail(W4_ERR_ARG, "sweep: unknown mode %d", mode);
    for (int i = 0; i < n_ops; ++i) {
        const int st = check_op(ops[i], i);
        if (st != W4_OK) return st;
    }
    {
        const int st = config_status();   // GRAPH mode picks each op's tile
        if (st != W4_OK) return st;
    }
    {
        const int st = check_outputs_spare_inputs(std::vector<w4_gemv_op>(ops, ops + n_ops));
        if (st != W4_OK) return st;
    }
    if (mode != W4_SWEEP_GRAPH) {
        for (int i = 0; i < n_ops; ++i)
            if (ops[i].K / 32 > kPwMaxC)
                return fail(W4_ERR_UNSUPPORTED,
                            "sweep op %d: persistent modes serve K <= %d (got %d)", i,
                            kPwMaxC * 32, ops[i].K);
    }
    w4_sweep* h = new (std::nothrow) w4_sweep;
    if (!h) return fail(W4_ERR_NOMEM, "sweep: host allocation failed");
    h->mode = mode;
    h->ops.assign(ops, ops + n_ops);
    for (const w4_gemv_op& op : h->ops)
        h->weight_bytes += (size_t)op.N * op.K / 2 + (size_t)op.N * (op.K / op.group) * 2;

    hipStream_t cs = nullptr;
    int st = hip_fail(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking), "sweep stream");
    if (st != W4_OK) {
        release(h);
        return st;
    }
    // GRAPH mode captures its per-op kernels into a graph.  The persistent
    // modes are one kernel each: it is launched directly (a one-node graph
    // launch costs more than the kernel launch it wraps); their op table and
    // control block are allocated and filled here.
    if (mode == W4_SWEEP_GRAPH) {
        st = hip_fail(hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal),
                      "begin capture");
        if (st == W4_OK) {
            const int cst = capture_graph_nodes(h, cs);
            const int est = hip_fail(hipStreamEndCapture(cs, &h->graph), "end capture");
            st = cst != W4_OK ? cst : est;
        }
        if (st == W4_OK)
            st = hip_fail(hipGraphInstantiate(&h->exec, h->graph, nullptr, nullptr, 0),
                          "graph instantiate");
    } else {
        st = setup_persistent(h);
        h->kernels = 1;
    }
    (void)hipStreamDestroy(cs);
    if (st != W4_OK) {
        release(h);
        return st;
    }
    *out = h;
    return W4_OK;
}

int w4_decode_sweep_launch(w4_sweep* h, void* stream) {
    if (!h) return fail(W4_ERR_ARG, "sweep: bad handle");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (h->mode != W4_SWEEP_GRAPH)
        return launch_persist(h->mode == W4_SWEEP_PERSISTENT,
                              static_cast<const SweepOp*>(h->dev), (int)h->ops.size(), h->ctl,
                              h->range, h->grid, h->first0, h->first1, h->pre,
                              h->poll_limit, s);
    if (!h->exec) return fail(W4_ERR_ARG, "sweep: bad handle");
    return hip_fail(hipGraphLaunch(h->exec, s), "graph launch");
}

int w4_decode_sweep_check(w4_sweep* h, void* stream) {
    if (!h) return fail(W4_ERR_ARG, "sweep: bad handle");
    int st = hip_fail(hipStreamSynchronize(static_cast<hipStream_t>(stream)), "sweep sync");
    if (st != W4_OK || !h->ctl) return st;
    unsigned err = 0;
    st = hip_fail(hipMemcpy(&err, &h->ctl->error, sizeof err, hipMemcpyDeviceToHost),
                  "sweep error word");
    if (st != W4_OK) return st;
    if (err != 0) {
        // a replay that gave up leaves its counters part-way: start over
        (void)hipMemset(h->ctl, 0, sweep_ctl_bytes(h->grid));
        (void)hipDeviceSynchronize();
        return fail(W4_ERR_TIMEOUT, "sweep: a bounded in-kernel wait gave up");
    }
    return W4_OK;
}

int w4_decode_sweep_info(const w4_sweep* h, int* n_ops, size_t* weight_bytes,
                         int* kernels_per_replay) {
    if (!h) return fail(W4_ERR_ARG, "sweep: bad handle");
    if (n_ops) *n_ops = (int)h->ops.size();
    if (weight_bytes) *weight_bytes = h->weight_bytes;
    if (kernels_per_replay) *kernels_per_replay = h->kernels;
    return W4_OK;
}

int w4_decode_sweep_destroy(w4_sweep* h) {
    if (!h) return fail(W4_ERR_ARG, "sweep: bad handle");
    release(h);
    return W4_OK;
}

}  // extern "C"
