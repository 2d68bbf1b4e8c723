#!/usr/bin/env python3
"""Benchmark: ms per decode-step weight sweep and its effective HBM GB/s.

One step = one replay of a decode step's weight sweep on one GPU: 35 decoder
layers x {qkv 2560x1536, o 1536x2048, gate_up 12288x1536, down 1536x6144}
plus the lm_head 262144x1536, int4 codes with bf16 scales per group of 32,
M = 1, 923,222,016 weight bytes, synthetic seeded weights and activations
(no trained weights).  Inputs are resident in HBM before timing.  GB/s counts
weight bytes with 1 GB = 1e9 B, the accounting of the pages' own figures
([P1] "Gemma 4 E2B on a 4 GB GPU with plain PyTorch, faster than llama.cpp",
summary line of the w4gemv.py kernel).

    python bench.py [--gpus 1] [--steps 200] [--warmup 50] [--mode auto]

Prints one JSON line.  The headline respects decode order: op i + 1 starts
only after every output of op i is written, as in a decode step ([P1],
paragraph on the step captured once as a graph and replayed per token).
Each step is one replay of a captured graph: the decode-ordered persistent
kernel captured as a one-node graph ("persistent"), or the 141 GEMV kernels
captured in order ("graph"); the default "auto" times both with the same
steps and reports the faster, naming it in config.mode.
ms_per_step is the median of five timed regions of --steps replays each.
Reported under "extra", labelled: the other ordered mode, direct launches
without a graph, and the 141 GEMVs with no ordering between them
("stream", an upper bound: no decode step can run its GEMVs unordered), plus
the other workloads' kernels.  The CPU baseline times the fp64 oracle on the
host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A16 GEMV effective HBM GB/s (% of peak) + ms per 35-layer+lm_head sweep"
PEAK_HBM_GBPS = 8000.0
MODES = {"graph": 0, "persistent": 1, "stream": 2}
ORDERED = ("persistent", "graph")
KERNEL_OF = {"persistent": "w4::ordered_kernel", "stream": "w4::stream_kernel"}
def log(msg):
    print(msg, file=sys.stderr, flush=True)


def load_traffic(kernel: str):
    """HBM bytes per launch of a sweep kernel from the committed counter
    summary, or None when it is missing or was taken on other kernel source."""
    from bit_weight_only_w4a16_amd import traffic
    try:
        with open(traffic.out_file(kernel)) as f:
            t = json.load(f)
    except (OSError, ValueError, KeyError):
        return None
    if t.get("kernel_source_hash") != traffic.kernel_source_hash(kernel):
        return None
    return t.get("hbm_bytes_per_launch")


def upload_sweep(torch, w4, synth, dev):
    cases = synth.decode_sweep()
    ops = []
    for c in cases:
        import numpy as np
        P = torch.from_numpy(c.P.view(np.int32)).to(dev)
        S = torch.from_numpy(c.S.view(np.int16)).to(dev)
        packed = w4.pack(P, S, c.N, c.K, c.group)
        del P, S
        x = torch.from_numpy(c.X[0].view(np.int16)).to(dev).view(torch.bfloat16)
        dt = torch.float32 if c.out_dtype == "f32" else torch.bfloat16
        y = torch.empty(c.N, dtype=dt, device=dev)
        ops.append((packed, c.N, c.K, c.group, x, y))
    torch.cuda.synchronize()
    return cases, ops


def time_steps(torch, step, steps, warmup, trials=5):
    """ms per step of `step()` (one replay): `warmup` untimed steps, then
    `trials` timed regions of `steps` steps, each between HIP events on the
    current stream with a device synchronize on both sides."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    out = []
    for _ in range(trials):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / steps)
    return out


def captured(torch, sw):
    """One launch of the sweep captured as a graph (replayed per step)."""
    for _ in range(3):
        sw.launch()
    sw.check()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sw.launch()
    torch.cuda.synchronize()
    return g


def trial_stats(ms_list):
    t = sorted(v * 1e3 for v in ms_list)
    med = t[len(t) // 2]
    return {"n": len(t), "median_us": med, "min_us": t[0], "max_us": t[-1],
            "spread_pct": (t[-1] - t[0]) / med * 100, "trials_us": [v * 1e3 for v in ms_list]}


def time_mode(torch, w4, ops, name, steps, warmup, direct=False):
    """Trials of one sweep mode.  graph: the 141-node graph (its launch is a
    graph launch); persistent, stream: one kernel launch, captured as a
    one-node graph unless direct."""
    sw = w4.DecodeSweep(ops, MODES[name])
    if name == "graph" or direct:
        step = sw.launch
        g = None
    else:
        g = captured(torch, sw)
        step = g.replay
    ms = time_steps(torch, step, steps, warmup)
    sw.check()
    info = sw.info()
    del g
    sw.close()
    return ms, info


def probe_read(torch, w4, dev, nbytes=4 << 30, reps=10):
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    out = torch.empty(1, dtype=torch.int32, device=dev)
    for _ in range(2):
        w4.probe_read(buf, out=out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        w4.probe_read(buf, out=out)
    e1.record()
    torch.cuda.synchronize()
    gbps = nbytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
    del buf
    torch.cuda.empty_cache()
    return gbps


def time_calls(torch, fn, calls=20, reps=10):
    """Microseconds per call of fn: `calls` calls captured in one graph,
    replayed `reps` times between HIP events (no host overhead per call)."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * calls) * 1e3


def time_gather(torch, w4, synth, dev, embed_packed):
    """Row lookup in the step's 4-bit tables, bf16 out: the token-embedding
    table (the lm_head's packed copy, 262144 x 1536) and the per-layer input
    table (262144 x 8960), for 1 token (decode) and 512 tokens (prefill)."""
    import numpy as np
    out = {}
    ple = synth.ple_table()
    P = torch.from_numpy(ple.P.view(np.int32)).to(dev)
    S = torch.from_numpy(ple.S.view(np.int16)).to(dev)
    ple_packed = w4.pack(P, S, ple.N, ple.K, ple.group)
    del P, S
    for name, packed, K in (("embed_262144x1536", embed_packed, synth.HIDDEN),
                            ("ple_262144x8960", ple_packed, synth.PLE_WIDTH)):
        for B in (1, 512):
            ids = torch.from_numpy(synth.token_ids(B, 7)).to(dev)
            Y = torch.empty((B, K), dtype=torch.bfloat16, device=dev)
            us = time_calls(torch, lambda: w4.gather(packed, synth.VOCAB, K, 32, ids, "bf16",
                                                     out=Y))
            moved = B * (K // 2 + K // 32 * 2) + B * K * 2
            out["%s_B%d" % (name, B)] = {"us": us, "GBps_read_plus_write": moved / us / 1e3}
    del ple_packed
    return out


def time_quantize(torch, w4, synth, dev):
    """Offline rotate-and-quantize of the prefill-shaped weight (12288 x 1536
    fp32 with outlier channels -> 512-point rotation, int4 group 256)."""
    N, K = 2 * 6144, synth.HIDDEN
    W = torch.from_numpy(synth.outlier_weights(N, K, 13)).to(dev)
    out = torch.empty(w4.packed_bytes(N, K, 256), dtype=torch.uint8, device=dev)
    us = time_calls(torch, lambda: w4.quantize(W, 256, 512, out=out))
    moved = N * K * 4 + w4.packed_bytes(N, K, 256)
    return {"shape": "12288x1536 fp32 -> g256, had_block 512", "us": us,
            "GBps_read_plus_write": moved / us / 1e3}


def time_attention(torch, w4, dev):
    """Split-K decode attention, 8 query heads on one KV head: full-length
    caches (head width 512) at 4096 / 32768 / 131072 slots, and a sliding
    layer's 512-slot ring (width 256).  Bytes = K and V of the slots scanned."""
    import numpy as np
    out = {}
    rng = np.random.default_rng(5)
    cases = [("full_D512_T4096", 512, 4096, False), ("full_D512_T32768", 512, 32768, False),
             ("full_D512_T131072", 512, 131072, False), ("ring_D256_S512", 256, 512, True)]
    for name, D, T, ring in cases:
        K = torch.randn((T, D), device=dev).to(torch.bfloat16)
        V = torch.randn((T, D), device=dev).to(torch.bfloat16)
        q = torch.randn((8, D), device=dev).to(torch.bfloat16)
        Vt = w4.attn_pack_v(V)
        pos = None
        cur = T - 1
        if ring:
            cur = 5000
            pos = torch.from_numpy(np.array([cur - ((cur - s) % T) for s in range(T)],
                                            dtype=np.int32)).to(dev)
        ws = torch.empty(w4.attn_workspace_bytes(T, D), dtype=torch.uint8, device=dev)
        o = torch.empty((8, D), dtype=torch.bfloat16, device=dev)
        us = time_calls(torch, lambda: w4.attn_decode(q, K, Vt, T, 1.0 / D ** 0.5, pos=pos,
                                                      cur=cur, window=512 if ring else 0,
                                                      out_dtype="bf16", out=o, workspace=ws))
        kv = 2 * T * D * 2
        out[name] = {"us": us, "kv_GBps": kv / us / 1e3, "pct_of_8TBps": kv / us / 1e3 / 80.0}
        del K, V, Vt, ws
    return out


def time_twin(torch, w4, synth, dev):
    """The auto:M switch on the prefill-shaped weight (12288 x 1536, rotated
    along K with 512-point blocks): int4 group 256 (w4a16_gemm with the
    run-time transform) against the int8 twin (activations rotated and
    quantized at run time, int8 matrix cores), bf16 out."""
    import numpy as np
    N, K = 2 * 6144, synth.HIDDEN
    W = torch.from_numpy(synth.outlier_weights(N, K, 13)).to(dev)
    packed4 = w4.quantize(W, 256, 512)
    W8, ws8 = w4.quantize_rows_i8(W, 512)
    del W
    out = {}
    for M in (8, 16, 64, 512):
        X = torch.from_numpy(synth.draw_activations(np.random.default_rng(M), M, K)
                             .view(np.int16)).to(dev).view(torch.bfloat16)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws4 = torch.empty(max(1, w4.gemm_workspace_bytes(M, K, 512)), dtype=torch.uint8,
                          device=dev)
        ws8b = torch.empty(max(1, int(w4.lib().w4a16_gemm_twin_workspace_bytes(M, K, 512, 1))),
                           dtype=torch.uint8, device=dev)
        int4_us = time_calls(torch, lambda: w4.gemm(packed4, N, K, 256, X, 512, "bf16", out=Y,
                                                    workspace=ws4))
        int8_us = time_calls(torch, lambda: w4.gemm_twin(packed4, W8, ws8, N, K, 256, X, 512, 1,
                                                         "bf16", out=Y, workspace=ws8b))
        auto_us = int8_us if M >= 16 else int4_us
        ops = 2.0 * M * N * K
        out["M%d" % M] = {"int4_us": int4_us, "int8_twin_us": int8_us,
                          "auto16_picks": "int8" if M >= 16 else "int4", "auto16_us": auto_us,
                          "int8_TOPS": ops / int8_us / 1e6,
                          "int8_pct_of_5POPS": ops / int8_us / 1e6 / 5000 * 100}
    return out


def time_mfma_probe(torch, w4):
    """Measured matrix-core ceiling: back-to-back independent bf16 MFMAs from
    registers at two waves per SIMD (w4_probe_mfma)."""
    iters = 512
    out = torch.zeros(1, dtype=torch.float32, device="cuda")
    us = time_calls(torch, lambda: w4.probe_mfma(iters, out), calls=10, reps=5)
    flops = 2048.0 * iters * 16 * 16384
    return {"iters": iters, "us": us, "TFLOPs": flops / us / 1e6,
            "pct_of_2.5PF_bf16": flops / us / 1e6 / 2500 * 100}


def time_handoff_probe(torch, w4):
    """The decode-ordered sweep's per-op handoff without weights
    (w4_probe_handoff): us per round from two round counts (launched
    directly, HIP events, median of five each), the difference over the extra
    rounds.  rows bf16 outputs per workgroup per round, and 256 * rows * 2
    bytes loaded by every workgroup: 6 rows = the 3 KB input of the K = 1536
    ops, 24 = the 12 KB input of the down projection, 48 = the gate+up output
    rows per workgroup.  handoff_floor_us: the handoffs of one step at these
    sizes (106 at 6 rows: three per layer and the lm_head's; 35 at 24)."""
    r1, r2 = 64, 1088
    work = w4.probe_handoff(1, 0)
    res = {"rounds": [r1, r2]}

    def once(rounds, rows):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        w4.probe_handoff(rounds, rows, work)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3

    for rows in (0, 6, 24, 48):
        once(r1, rows)
        t = {}
        for r in (r1, r2):
            v = sorted(once(r, rows) for _ in range(5))
            t[r] = v[2]
        if int(work[:4].view(torch.int32).item()) != 0:
            raise RuntimeError("handoff probe: a poll gave up")
        res["rows%d_us_per_round" % rows] = (t[r2] - t[r1]) / (r2 - r1)
    res["handoff_floor_us"] = (106 * res["rows6_us_per_round"] +
                               35 * res["rows24_us_per_round"])
    return res


def time_prefill(torch, w4, synth, dev, mfma_tflops=None):
    """The prefill-shaped product, group 256, N=12288, K=1536 with the 512-point
    run-time Hadamard transform, at M = 8 (small-M kernel), 64 and 512 (matrix
    cores); also the transform alone, the product without it, and, for
    context, torch's dense bf16 matmul of the same shape."""
    import numpy as np
    out = {}
    for M in (8, 64, 512):
        c = synth.prefill_g256(M)
        P = torch.from_numpy(c.P.view(np.int32)).to(dev)
        S = torch.from_numpy(c.S.view(np.int16)).to(dev)
        packed = w4.pack(P, S, c.N, c.K, c.group)
        X = torch.from_numpy(c.X.view(np.int16)).to(dev).view(torch.bfloat16)
        Y = torch.empty((M, c.N), dtype=torch.bfloat16, device=dev)
        Xr = torch.empty_like(X)
        ws = torch.empty(max(1, w4.gemm_workspace_bytes(M, c.K, 512)), dtype=torch.uint8,
                         device=dev)
        res = {"kernel": w4.describe_dispatch(M, c.N, c.K, c.group)}
        res["fwht_plus_gemm_us"] = time_calls(torch, lambda: w4.gemm(
            packed, c.N, c.K, c.group, X, 512, "bf16", out=Y, workspace=ws))
        res["gemm_us"] = time_calls(torch, lambda: w4.gemm(
            packed, c.N, c.K, c.group, X, 0, "bf16", out=Y))
        res["fwht_us"] = time_calls(torch, lambda: w4.fwht(X, 512, out=Xr))
        flops = 2.0 * M * c.N * c.K
        t = res["gemm_us"] * 1e-6
        res["gemm_TFLOPs"] = flops / t / 1e12
        res["gemm_pct_of_2.5PF_bf16"] = flops / t / 2.5e15 * 100
        if mfma_tflops:
            res["gemm_pct_of_mfma_probe"] = flops / t / 1e12 / mfma_tflops * 100
        res["gemm_weight_GBps"] = c.weight_bytes / t / 1e9
        # context, not a target: the vendor library's dense bf16 GEMM of the
        # same shape (torch.matmul, hipBLASLt), with 16-bit weights (4x the
        # bytes) and no decode
        Wd = torch.randn(c.N, c.K, device=dev, dtype=torch.bfloat16)
        us = time_calls(torch, lambda: torch.matmul(X, Wd.t(), out=Y))
        res["dense_bf16_matmul_us"] = us
        res["dense_bf16_matmul_pct_of_2.5PF"] = flops / (us * 1e-6) / 2.5e15 * 100
        out["M%d" % M] = res
        del P, S, packed, X, Y, Xr, ws, Wd
    torch.cuda.empty_cache()
    return out


def time_gemm_shapes(torch, w4, synth, dev, N, K, group, Ms):
    """The W4A16 product alone (no transform), bf16 out, at one weight shape
    and several row counts: the down projection (N = 1536, K = 6144) and the
    group-32 form of the gate+up shape."""
    import numpy as np
    out = {}
    for M in Ms:
        c = synth.make_case("gemm_%dx%d_g%d_M%d" % (N, K, group, M), N, K, group, M,
                            2000 + M, "bf16", outlier_frac=0.01)
        P = torch.from_numpy(c.P.view(np.int32)).to(dev)
        S = torch.from_numpy(c.S.view(np.int16)).to(dev)
        packed = w4.pack(P, S, N, K, group)
        X = torch.from_numpy(c.X.view(np.int16)).to(dev).view(torch.bfloat16)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        us = time_calls(torch, lambda: w4.gemm(packed, N, K, group, X, 0, "bf16", out=Y))
        flops = 2.0 * M * N * K
        out["M%d" % M] = {"kernel": w4.describe_dispatch(M, N, K, group), "gemm_us": us,
                          "gemm_TFLOPs": flops / us / 1e6,
                          "gemm_pct_of_2.5PF_bf16": flops / us / 1e6 / 2500 * 100}
        del P, S, packed, X, Y
    torch.cuda.empty_cache()
    return out


def time_single_gemv(torch, w4, synth, dev, cases, ops):
    """The single-GEMV workloads, batch 1: the 256 x 512 case, the four
    decoder-layer shapes (layer 0 of the sweep) and the 262144 x 1536
    lm_head.  Warm: 20 calls on one copy, graph-replayed.  Cold: one call on
    each of at least 1 GiB of distinct device copies of the same packed
    matrix (the copies count is reported), so the 256 MB last-level cache
    holds none of them when its turn comes.  The 256 x 512 case (73 KB) is
    latency-bound and reported warm only."""
    import numpy as np
    out = {}
    c1 = synth.make_case("single", 256, 512, 32, 1, 0, "f32")
    P = torch.from_numpy(c1.P.view(np.int32)).to(dev)
    S = torch.from_numpy(c1.S.view(np.int16)).to(dev)
    p1 = w4.pack(P, S, 256, 512, 32)
    x1 = torch.from_numpy(c1.X[0].view(np.int16)).to(dev).view(torch.bfloat16)
    y1 = torch.empty(256, dtype=torch.float32, device=dev)
    out["256x512_g32"] = {"warm_us": time_calls(torch, lambda: w4.gemv(p1, 256, 512, 32, x1,
                                                                        "f32", out=y1))}
    del P, S, p1
    for idx in (0, 1, 2, 3, len(ops) - 1):
        packed, N, K, g, x, y = ops[idx]
        odt = "f32" if y.dtype == torch.float32 else "bf16"
        name = "%s_%dx%d" % (cases[idx].name.split("_seed")[0], N, K)
        res = {"warm_us": time_calls(torch, lambda: w4.gemv(packed, N, K, g, x, odt, out=y))}
        nbytes = cases[idx].weight_bytes
        n = int(max(2, -(-(1 << 30) // packed.numel())))
        copies = [packed.clone() for _ in range(n)]
        it = iter(range(1 << 30))
        res["cold_us"] = time_calls(torch, lambda: w4.gemv(copies[next(it) % n], N, K, g, x, odt,
                                                              out=y), calls=n, reps=3)
        res["cold_copies"] = n
        res["cold_GBps"] = nbytes / res["cold_us"] / 1e3
        res["warm_GBps"] = nbytes / res["warm_us"] / 1e3
        out[name] = res
        del copies
        torch.cuda.empty_cache()
    return out


def time_smallm_g32(torch, w4, synth, dev):
    """A few rows through the decode-format (group 32) gate+up weight,
    12288 x 1536, at 2, 8, 16 and 32 rows, bf16 out: w4a16_gemm (whatever it
    dispatches to, named in "kernel") and, to 16 rows, the small-M entry
    point (w4a16_gemm_smallM, its own kernels)."""
    import numpy as np
    c = synth.make_case("smallm_g32", 12288, 1536, 32, 32, 16, "bf16")
    P = torch.from_numpy(c.P.view(np.int32)).to(dev)
    S = torch.from_numpy(c.S.view(np.int16)).to(dev)
    packed = w4.pack(P, S, c.N, c.K, c.group)
    X16 = torch.from_numpy(c.X.view(np.int16)).to(dev).view(torch.bfloat16)
    out = {}
    for M in (2, 8, 16, 32):
        X = X16[:M]
        Y = torch.empty((M, c.N), dtype=torch.bfloat16, device=dev)
        us = time_calls(torch, lambda: w4.gemm(packed, c.N, c.K, c.group, X, 0, "bf16", out=Y))
        r = {"kernel": w4.describe_dispatch(M, c.N, c.K, c.group), "us": us,
             "weight_GBps": c.weight_bytes / us / 1e3}
        if M <= 16:
            r["smallM_entry_us"] = time_calls(torch, lambda: w4.gemm_smallM(
                packed, c.N, c.K, c.group, X, "bf16", out=Y))
        out["M%d" % M] = r
    del P, S, packed, X16
    return out


def host_threads():
    """Threads for the CPU baseline: every core this process may run on,
    capped by OMP_NUM_THREADS when it is set (a shared host's CPU share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_baseline(cases, max_threads=None, min_seconds=10.0, max_passes=40):
    """The fp64 oracle over whole decode-step sweeps (all 141 GEMVs), OpenMP
    over rows on the host's cores, repeated until min_seconds of wall time (at
    most max_passes): a bounded sample of about 10 s."""
    import oracle
    oracle.build()
    threads = host_threads() if max_threads is None else max(1, max_threads)
    total = 0
    passes = 0
    t0 = time.perf_counter()
    while passes < max_passes:
        for c in cases:
            oracle.gemm_bf16(c.P, c.S, c.N, c.K, c.group, c.X[0], threads=threads)
            total += c.weight_bytes
        passes += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": total / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "nproc": os.cpu_count(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "sample": "%d full decode-step sweep(s) (141 GEMVs, %d weight bytes each) in "
                      "%.1f s with the scalar fp64 oracle on %d threads (nproc %s)"
                      % (passes, total // passes, dt, threads, os.cpu_count())}


def cpu_oracle_per_config(synth, cases, threads):
    """The fp64 oracle on each workload, one host thread and `threads`
    threads, median of three wall times (perf_counter) per entry: the
    256 x 512 GEMV, decoder layer 0's four GEMVs, the lm_head GEMV, and the
    prefill product with its 512-point transform at 8 rows (64 and 512 rows
    given as that time scaled, the oracle being linear in the rows)."""
    import oracle
    oracle.build()
    import numpy as np

    def med3(fn):
        t = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn()
            t.append(time.perf_counter() - t0)
        return sorted(t)[1]

    out = {"threads": threads, "nproc": os.cpu_count(), "timing": "median of 3, perf_counter"}
    c1 = synth.make_case("single", 256, 512, 32, 1, 0, "f32")
    gemv_sets = (("256x512_g32", [c1]), ("decoder_layer_4_gemvs", cases[:4]),
                 ("lm_head_262144x1536", [cases[-1]]))
    for name, cs in gemv_sets:
        wb = sum(c.weight_bytes for c in cs)
        r = {"weight_bytes": wb}
        for label, th in (("one_thread", 1), ("all_threads", threads)):
            dt = med3(lambda: [oracle.gemm_bf16(c.P, c.S, c.N, c.K, c.group, c.X[0], threads=th)
                               for c in cs])
            r[label + "_ms"] = dt * 1e3
            r[label + "_GBps"] = wb / dt / 1e9
        out[name] = r
    # the oracle's time is linear in the rows: the 8-row product is timed,
    # 64 and 512 rows are that time scaled
    c = synth.prefill_g256(8)
    x = oracle.bf16_to_f64(c.X)
    flops = 2.0 * 8 * c.N * c.K
    r = {"rows_timed": 8}
    for label, th in (("one_thread", 1), ("all_threads", threads)):
        dt = med3(lambda: oracle.gemm(c.P, c.S, c.N, c.K, c.group, oracle.fwht(x, 512),
                                      threads=th))
        r[label + "_GFLOPs"] = flops / dt / 1e9
        for M in (8, 64, 512):
            r[label + "_ms_M%d" % M] = dt * 1e3 * M / 8
    out["prefill_g256_N12288_K1536"] = r
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--mode", choices=sorted(MODES) + ["auto"], default="auto",
                    help="headline mode: auto (default) = the faster of the two "
                         "decode-ordered modes, persistent (one kernel) and graph (141 "
                         "kernels); stream = the unordered upper bound (for counter runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--handoff-only", action="store_true",
                    help="time only the grid-wide handoff probe and print its JSON")
    ap.add_argument("--kernel-only", action="store_true",
                    help="for hardware-counter runs: only --steps replays of the timed "
                         "mode, then three 1 GiB probe copies (the calibration kernel); "
                         "prints nothing")
    ap.add_argument("--prefill-only", type=int, default=0, metavar="M",
                    help="for hardware-counter runs: only --steps calls of the prefill "
                         "product (group 256, N=12288, K=1536, no transform) at M rows; "
                         "prints nothing")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU; this library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_weight_only_w4a16_amd as w4
    from bit_weight_only_w4a16_amd import synth

    dev = torch.device("cuda:0")
    w4.device_check()
    if args.handoff_only:
        print(json.dumps(time_handoff_probe(torch, w4)))
        return
    if args.prefill_only:
        import numpy as np
        c = synth.prefill_g256(args.prefill_only)
        P = torch.from_numpy(c.P.view(np.int32)).to(dev)
        S = torch.from_numpy(c.S.view(np.int16)).to(dev)
        packed = w4.pack(P, S, c.N, c.K, c.group)
        X = torch.from_numpy(c.X.view(np.int16)).to(dev).view(torch.bfloat16)
        Y = torch.empty((c.M, c.N), dtype=torch.bfloat16, device=dev)
        for _ in range(args.steps):
            w4.gemm(packed, c.N, c.K, c.group, X, 0, "bf16", out=Y)
        torch.cuda.synchronize()
        return
    log("generating and packing the sweep")
    cases, ops = upload_sweep(torch, w4, synth, dev)
    weight_bytes = sum(c.weight_bytes for c in cases)
    io_bytes = sum(c.K * 2 + c.N * (4 if c.out_dtype == "f32" else 2) for c in cases)

    if args.kernel_only:
        # one kernel per step: the persistent kernels only
        mode = "persistent" if args.mode in ("auto", "graph") else args.mode
        sw = w4.DecodeSweep(ops, MODES[mode])
        for _ in range(args.steps):
            sw.launch()
        sw.check()
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        for _ in range(3):
            w4.probe_copy(src, dst)
        torch.cuda.synchronize()
        sw.close()
        return

    extra = {}
    # the read probe and the other modes run first; they also bring the GPU
    # out of idle before the headline's warm-up
    probe = probe_read(torch, w4, dev) if not args.no_extra else None
    head_modes = list(ORDERED) if args.mode == "auto" else [args.mode]
    modes = {}
    side = 20
    if not args.no_extra:
        for name in ("graph", "persistent", "stream"):
            if name in head_modes:
                continue
            ms, _ = time_mode(torch, w4, ops, name, side, 5)
            modes[name] = trial_stats(ms)
        for name in ("persistent", "stream"):
            ms, _ = time_mode(torch, w4, ops, name, side, 5, direct=True)
            modes[name + "_direct_launch"] = trial_stats(ms)
    head = {}
    for name in head_modes:
        ms, info = time_mode(torch, w4, ops, name, args.steps, args.warmup)
        head[name] = (ms, info)
        modes[name] = trial_stats(ms)
        log("%-10s median %.1f us/step" % (name, modes[name]["median_us"]))
    mode = min(head, key=lambda m: modes[m]["median_us"])
    ms = modes[mode]["median_us"] / 1e3
    kernels = head[mode][1]["kernels"]
    value = weight_bytes / (ms * 1e-3) / 1e9
    for name, t in modes.items():
        t["GBps"] = weight_bytes / (t["median_us"] * 1e-6) / 1e9
        t["pct_of_8TBps"] = t["GBps"] / PEAK_HBM_GBPS * 100
        t["decode_ordered"] = not name.startswith("stream")
        t["graph_captured"] = not name.endswith("_direct_launch")

    if not args.no_extra:
        mfma = time_mfma_probe(torch, w4)
        extra = {
            "pct_of_8TBps_spec": value / PEAK_HBM_GBPS * 100,
            "probe_read_4GiB_GBps": probe,
            "GBps_incl_x_y": (weight_bytes + io_bytes) / (ms * 1e-3) / 1e9,
            "ms_per_1222.8MiB_at_this_rate": 1282203648 / (value * 1e9) * 1e3,
            "modes": modes,
            "stream_upper_bound_note": "stream: the 141 GEMVs with no ordering between them "
                                       "(one kernel, graph-captured); no decode step can run "
                                       "unordered, so it bounds what ordering costs",
            "single_gemv": time_single_gemv(torch, w4, synth, dev, cases, ops),
            "mfma_probe": mfma,
            "handoff_probe": time_handoff_probe(torch, w4),
            "prefill_g256_N12288_K1536": time_prefill(torch, w4, synth, dev, mfma["TFLOPs"]),
            "prefill_down_g256_N1536_K6144": time_gemm_shapes(torch, w4, synth, dev, 1536,
                                                              6144, 256, (64, 512)),
            "prefill_g32_N12288_K1536": time_gemm_shapes(torch, w4, synth, dev, 12288, 1536,
                                                         32, (64, 512)),
            "smallm_g32_N12288_K1536": time_smallm_g32(torch, w4, synth, dev),
            "gather_bf16": time_gather(torch, w4, synth, dev, ops[-1][0]),
            "quantize_rotate": time_quantize(torch, w4, synth, dev),
            "int8_twin_auto16": time_twin(torch, w4, synth, dev),
            "attention_decode": time_attention(torch, w4, dev),
        }
        if "stream" in modes:
            st = modes["stream"]
            extra["stream_roofline"] = {
                "kernel": KERNEL_OF["stream"], "achieved": st["GBps"], "peak": PEAK_HBM_GBPS,
                "frac": st["GBps"] / PEAK_HBM_GBPS, "traffic": load_traffic("stream")}

    # Roofline of the step's dominant kernel.  persistent: the step is one
    # kernel, so bytes per launch / replay time (HIP events on the stream the
    # graph is replayed on; the replay adds the graph launch to the kernel).
    # graph: 141 kernels per step (the largest, the lm_head GEMV, takes ~6 %
    # of the step), none dominant: the step's bytes / step time.
    achieved = weight_bytes / (ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBPS,
                "traffic": load_traffic(mode) if mode in KERNEL_OF else None,
                "kernel": KERNEL_OF.get(mode, "141 GEMV kernels (whole step)")}

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on one sweep")
        cpu = cpu_baseline(cases)
        if not args.no_extra:
            # the same oracle on one host thread, on decoder layer 0's four
            # GEMVs (19.9 MB), scaled to a whole sweep
            one = cpu_baseline(cases[:4], max_threads=1, min_seconds=1.0, max_passes=5)
            extra["cpu_oracle_one_thread"] = {
                "GBps": one["value"], "sample": one["sample"].replace(
                    "full decode-step sweep(s) (141 GEMVs", "pass(es) over decoder layer 0 (4 GEMVs"),
                "ms_per_sweep_scaled": weight_bytes / one["value"] / 1e6}
            log("timing the CPU oracle on each workload")
            extra["cpu_oracle_per_config"] = cpu_oracle_per_config(synth, cases, cpu["cores"])

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "decode-step weight sweep: 35 x {qkv 2560x1536, o 1536x2048, "
                        "gate_up 12288x1536, down 1536x6144} + lm_head 262144x1536, "
                        "int4 group-32 bf16 scales, M=1, fresh seed per matrix",
            "weight_bytes": weight_bytes,
            "ops": len(cases),
            "mode": mode,
            "decode_ordered": mode != "stream",
            "graph_captured": True,
            "kernels_per_step": kernels,
            "ms_per_step_is": "median of 5 timed regions of --steps replays",
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
