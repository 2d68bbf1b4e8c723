"""Offline search for the batch-1 GEMV tile table on the current GPU.

[P1] "Gemma 4 E2B on a 4 GB GPU with plain PyTorch, faster than llama.cpp",
paragraph on the w4gemv.py kernel: each weight shape gets its own fixed
tiling, chosen by searching tile sizes, warps and pipeline stages on the card.

For each shape, every legal tile (lanes per row L with U = ceil(K / 32 / L)
chunks per lane, waves per workgroup, grid, pipeline stages, strided or
contiguous rows; and the generic loop) is loaded as a one-line table
(w4_tile_table_load) and timed cold: one call per distinct copy of the packed
matrix, the copies together at least 1 GiB so that the 256 MB last-level
cache holds none of them when its turn comes, all calls captured in one graph
and replayed.  A candidate whose output strays from the heuristic tile's
output by more than 1e-3 of its largest magnitude stops the search with an
error: a tile the table accepts must compute the product (the GPU parity
tests check every tile path against the oracle).  The fastest
candidate per shape goes to the table, with the heuristic's time beside it:
the five fastest of the first pass and the heuristic are timed five more
times each, interleaved, and the lowest median wins (the heuristic keeps the
shape when it is fastest).

    python -m bit_weight_only_w4a16_amd.tune --out tiles_mi355x.txt
    python -m bit_weight_only_w4a16_amd.tune --header tiles_mi355x.txt csrc/w4_tiles.h

Default shapes: the model's decode GEMVs (256 x 512; q/k/v 2560 x 1536,
o 1536 x 2048, gate+up 12288 x 1536, down 1536 x 6144; lm_head 262144 x 1536;
group 32).
"""
import argparse
import os
import sys
import time

SHAPES = [(256, 512, 32, "f32"), (2560, 1536, 32, "bf16"), (1536, 2048, 32, "bf16"),
          (12288, 1536, 32, "bf16"), (1536, 6144, 32, "bf16"), (262144, 1536, 32, "f32")]
GRIDS = (64, 128, 256, 512, 1024, 2048, 4096)
CONTIG_GRIDS = (256, 512, 1024, 2048)


def candidates(N, K, group):
    """(L, U, waves, grid, stages, contig) tuples the table format accepts."""
    C = K // 32
    out = []
    tiled = (K // group) % 2 == 0
    for L in (8, 16, 32, 64):
        U = (C + L - 1) // L
        if not tiled or U > 8:
            continue
        NG = (N + 64 // L - 1) // (64 // L)
        for waves in (1, 2, 4):
            cap = (NG + waves - 1) // waves
            grids = [0] + [g for g in GRIDS if g < cap]
            for grid in grids:
                for stages in ((2, 3) if U <= 4 else (2,)):
                    out.append((L, U, waves, grid, stages, 0))
        if L >= 16 and L * U == C and U <= 3:
            for grid in [0] + list(CONTIG_GRIDS):
                for stages in (2, 3):
                    out.append((L, U, 4, grid, stages, 1))
    for L in (16, 64):
        out.append((L, 0, 4, 0, 2, 0))
    return out


def entry(N, K, group, c):
    return "gemv %d %d %d %d %d %d %d %d %d" % ((N, K, group) + tuple(c))


def time_cold(torch, w4, copies, N, K, group, x, y, odt, reps=3):
    """Microseconds per call, one call per copy, captured in one graph."""
    for p in copies[:2]:
        w4.gemv(p, N, K, group, x, odt, out=y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for p in copies:
            w4.gemv(p, N, K, group, x, odt, out=y)
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / (reps * len(copies)) * 1e3


def search(shapes, log=print):
    import numpy as np
    import torch
    import bit_weight_only_w4a16_amd as w4
    from bit_weight_only_w4a16_amd import synth
    w4.device_check()
    dev = torch.device("cuda:0")
    tmp = os.path.join(os.environ.get("TMPDIR", "/tmp"), "w4_tune_%d.txt" % os.getpid())
    props = torch.cuda.get_device_properties(0)
    lines = ["# batch-1 GEMV tile table for %s (%d CUs), searched by "
             "bit_weight_only_w4a16_amd.tune" % (props.gcnArchName.split(":")[0],
                                                props.multi_processor_count),
             "# gemv N K group L U waves grid stages contig   # cold us: best, heuristic"]
    try:
        for N, K, group, odt in shapes:
            c = synth.make_case("tune", N, K, group, 1, 1000 + N % 977, odt)
            P = torch.from_numpy(c.P.view(np.int32)).to(dev)
            S = torch.from_numpy(c.S.view(np.int16)).to(dev)
            packed = w4.pack(P, S, N, K, group)
            del P, S
            n = int(max(2, -(-(1 << 30) // packed.numel())))
            copies = [packed] + [packed.clone() for _ in range(n - 1)]
            x = torch.from_numpy(c.X[0].view(np.int16)).to(dev).view(torch.bfloat16)
            y = torch.empty(N, dtype=torch.float32 if odt == "f32" else torch.bfloat16,
                            device=dev)
            w4.tile_table_load(None)
            ref = w4.gemv(packed, N, K, group, x, odt).float().cpu().numpy()
            tol = 1e-3 * float(np.abs(ref).max()) + 1e-30
            t0 = time.time()
            cands = candidates(N, K, group)

            def load(cand):
                if cand is None:
                    w4.tile_table_load(None)
                    return
                with open(tmp, "w") as f:
                    f.write(entry(N, K, group, cand) + "\n")
                w4.tile_table_load(tmp)

            timed = []
            for cand in cands:
                load(cand)
                got = w4.gemv(packed, N, K, group, x, odt).float().cpu().numpy()
                if not np.all(np.abs(got - ref) <= tol):
                    raise RuntimeError("%s: output differs from the heuristic tile's"
                                       % entry(N, K, group, cand))
                timed.append((time_cold(torch, w4, copies, N, K, group, x, y, odt), cand))
            # the five fastest and the heuristic again, interleaved, five times:
            # the median decides (one fast run among many is not a win)
            finalists = [None] + [c for _, c in sorted(timed, key=lambda t: t[0])[:5]]
            runs = {c: [] for c in finalists}
            for _ in range(5):
                for cand in finalists:
                    load(cand)
                    runs[cand].append(time_cold(torch, w4, copies, N, K, group, x, y, odt,
                                                reps=5))
            med = {c: sorted(v)[2] for c, v in runs.items()}
            base = med[None]
            best = min(((med[c], c) for c in finalists), key=lambda t: t[0])
            w4.tile_table_load(None)
            log("%d x %d g%d: heuristic %.2f us, best %.2f us %s (%d candidates, %.0f s)"
                % (N, K, group, base, best[0], best[1], len(cands), time.time() - t0))
            if best[1] is not None:
                lines.append("%s   # %.2f %.2f" % (entry(N, K, group, best[1]), best[0], base))
            else:
                lines.append("# %d %d %d: the heuristic tile is fastest (%.2f us)"
                             % (N, K, group, base))
            del copies, packed
            torch.cuda.empty_cache()
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)
    return "\n".join(lines) + "\n"


def header(table_path):
    """C++ for csrc/w4_tiles.h from a table file (validated by the library)."""
    import bit_weight_only_w4a16_amd as w4
    w4.tile_table_load(table_path)   # raises on a malformed table
    w4.tile_table_load(None)
    rows = []
    for line in open(table_path):
        line = line.split("#", 1)[0].split()
        if not line:
            continue
        N, K, g, L, U, W, grid, st, ct = (int(v) for v in line[1:])
        rows.append("    {%d, %d, %d, GemvTile{%d, %d, %d, %d, %d, %s, %s}},"
                    % (N, K, g, L, U, W, grid, st, "true" if U == 0 else "false",
                       "true" if ct else "false"))
    n = len(rows)
    body = "\n".join(rows) if rows else "    {0, 0, 0, GemvTile{}},"
    return ("// w4_tiles.h -- the built-in GEMV tile table (included by w4_gemv.hip).\n"
            "// Written by `python -m bit_weight_only_w4a16_amd.tune --header` from\n"
            "// %s (searched on MI355X; the file's comments give\n"
            "// the cold time of each entry and of the heuristic tile).\n"
            "constexpr int kBuiltinTileCount = %d;\n"
            "static const TileEntry kBuiltinTiles[%d] = {\n%s\n};\n"
            % (os.path.basename(table_path), n, max(n, 1), body))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--out", help="write the searched table here")
    ap.add_argument("--header", nargs=2, metavar=("TABLE", "HEADER"),
                    help="write the built-in table header from a table file")
    args = ap.parse_args(argv)
    if args.header:
        text = header(args.header[0])
        with open(args.header[1], "w") as f:
            f.write(text)
        return 0
    text = search(SHAPES, log=lambda m: print(m, flush=True))
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    sys.stdout.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
