// w4_sweep.hip -- one decode step's GEMVs replayed as a single graph.
//
// [P1] "Gemma 4 E2B on a 4 GB GPU with plain PyTorch, faster than llama.cpp",
// paragraph on the decode step: hundreds of small kernels launched one at a
// time cost more than running them, so the step is captured once as a graph
// and replayed for every token.
#include <cstdlib>
#include <new>
#include <vector>

#include "w4_dispatch.h"

struct w4_sweep {
    int mode = 0;
    std::vector<w4_gemv_op> ops;
    size_t weight_bytes = 0;
    int kernels = 0;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
};

namespace w4 {

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

static int check_op(const w4_gemv_op& op, int i) {
    if (op.group != 32 && op.group != 256)
        return fail(W4_ERR_SHAPE, "sweep op %d: group must be 32 or 256", i);
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

static void release(w4_sweep* h) {
    if (h->exec) (void)hipGraphExecDestroy(h->exec);
    if (h->graph) (void)hipGraphDestroy(h->graph);
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
    if (mode != W4_SWEEP_GRAPH)
        return fail(W4_ERR_UNSUPPORTED, "sweep: persistent modes are not built yet");
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
    st = hip_fail(hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal), "begin capture");
    if (st == W4_OK) {
        const int cst = capture_graph_nodes(h, cs);
        const int est = hip_fail(hipStreamEndCapture(cs, &h->graph), "end capture");
        st = cst != W4_OK ? cst : est;
    }
    if (st == W4_OK)
        st = hip_fail(hipGraphInstantiate(&h->exec, h->graph, nullptr, nullptr, 0),
                      "graph instantiate");
    (void)hipStreamDestroy(cs);
    if (st != W4_OK) {
        release(h);
        return st;
    }
    *out = h;
    return W4_OK;
}

int w4_decode_sweep_launch(w4_sweep* h, void* stream) {
    if (!h || !h->exec) return fail(W4_ERR_ARG, "sweep: bad handle");
    return hip_fail(hipGraphLaunch(h->exec, static_cast<hipStream_t>(stream)), "graph launch");
}

int w4_decode_sweep_check(w4_sweep* h, void* stream) {
    if (!h) return fail(W4_ERR_ARG, "sweep: bad handle");
    return hip_fail(hipStreamSynchronize(static_cast<hipStream_t>(stream)), "sweep sync");
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
