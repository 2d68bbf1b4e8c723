"""HBM traffic of a decode-step sweep kernel from two hardware-counter runs.

    cd /tmp && TMPDIR=/tmp rocprofv3 --pmc FETCH_SIZE --output-format csv \
        -d <out>/pmc_fetch -o fetch -- python3 <repo>/bench.py --kernel-only \
        --mode <persistent|stream> --steps 20
    cd /tmp && TMPDIR=/tmp rocprofv3 --pmc WRITE_SIZE --output-format csv \
        -d <out>/pmc_write -o write -- python3 <repo>/bench.py --kernel-only \
        --mode <persistent|stream> --steps 20
    python -m bit_weight_only_w4a16_amd.traffic <persistent|stream> \
        <out>/pmc_fetch <out>/pmc_write

`bench.py --kernel-only` runs the mode's kernel, then three plain 1 GiB copies
(`w4_probe_copy`).  FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by
what they read for the copy, whose bytes are known, and the result is written
to profiles/traffic_sweep_<mode>.json together with a hash of the kernel's
source files: bench.py reports the figure only while that hash still matches.
"""
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_COMMON = ("bit_weight_only_w4a16_amd/csrc/w4_persist.h",
           "bit_weight_only_w4a16_amd/csrc/w4_gemv_core.h",
           "bit_weight_only_w4a16_amd/csrc/w4_common.h",
           "bit_weight_only_w4a16_amd/csrc/w4_sweep.hip")
SWEEP_KERNELS = {
    "stream": ("w4::stream_kernel",
               ("bit_weight_only_w4a16_amd/csrc/w4_persist.hip",) + _COMMON),
    "persistent": ("w4::ordered_kernel",
                   ("bit_weight_only_w4a16_amd/csrc/w4_ordered.hip",
                    "bit_weight_only_w4a16_amd/csrc/w4_ring.h") + _COMMON),
}
COPY_KERNEL = "w4::probe_copy_kernel"
COPY_BYTES = 1 << 30


def out_file(mode: str) -> str:
    SWEEP_KERNELS[mode]
    return os.path.join(ROOT, "profiles", "traffic_sweep_%s.json" % mode)


def kernel_source_hash(mode: str) -> str:
    h = hashlib.sha256()
    for rel in SWEEP_KERNELS[mode][1]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _counter_means(path: str, counter: str, kernel: str):
    """Mean counter value (KiB) per dispatch of the kernel and of the copy."""
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no *counter_collection.csv under %s" % path)
    vals = {kernel: [], COPY_KERNEL: []}
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                for k in vals:
                    if row["Kernel_Name"].startswith(k + "("):
                        vals[k].append(float(row["Counter_Value"]))
    for k, v in vals.items():
        if not v:
            raise SystemExit("no %s dispatch of %s in %s" % (counter, k, path))
    return ({k: sum(v) / len(v) for k, v in vals.items()},
            {k.split("::")[1]: len(v) for k, v in vals.items()})


def main(argv):
    if len(argv) != 4 or argv[1] not in SWEEP_KERNELS:
        raise SystemExit(__doc__)
    mode = argv[1]
    KERNEL = SWEEP_KERNELS[mode][0]
    fetch, n_fetch = _counter_means(argv[2], "FETCH_SIZE", KERNEL)
    write, _ = _counter_means(argv[3], "WRITE_SIZE", KERNEL)
    fetch_scale = COPY_BYTES / 1024.0 / fetch[COPY_KERNEL]
    write_scale = COPY_BYTES / 1024.0 / write[COPY_KERNEL]
    sys.path.insert(0, ROOT)
    from bit_weight_only_w4a16_amd import synth
    from bit_weight_only_w4a16_amd.accounting import weight_bytes as wbytes
    weight_bytes = (synth.N_LAYERS * sum(wbytes(N, K, 32) for _, N, K in synth.LAYER_SHAPES)
                    + wbytes(synth.LM_HEAD_SHAPE[1], synth.LM_HEAD_SHAPE[2], 32))
    hbm = fetch[KERNEL] * 1024.0 * fetch_scale + write[KERNEL] * 1024.0 * write_scale
    out = {
        "kernel": KERNEL,
        "kernel_source_hash": kernel_source_hash(mode),
        "hbm_bytes_per_launch": int(round(hbm)),
        "algorithmic_weight_bytes_per_launch": weight_bytes,
        "fetch_kib_per_dispatch": fetch[KERNEL],
        "write_kib_per_dispatch": write[KERNEL],
        "copy_calibration": {
            "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
            "fetch_kib_per_dispatch": fetch[COPY_KERNEL],
            "write_kib_per_dispatch": write[COPY_KERNEL],
            "fetch_scale": fetch_scale, "write_scale": write_scale,
        },
        "commands": [
            "cd /tmp && TMPDIR=/tmp timeout -s KILL 150 rocprofv3 --pmc FETCH_SIZE "
            "--output-format csv -d <out>/pmc_fetch -o fetch -- python3 <repo>/bench.py "
            "--kernel-only --mode %s --steps 20" % mode,
            "cd /tmp && TMPDIR=/tmp timeout -s KILL 150 rocprofv3 --pmc WRITE_SIZE "
            "--output-format csv -d <out>/pmc_write -o write -- python3 <repo>/bench.py "
            "--kernel-only --mode %s --steps 20" % mode,
            "python -m bit_weight_only_w4a16_amd.traffic %s <out>/pmc_fetch <out>/pmc_write"
            % mode,
        ],
        "dispatches": n_fetch,
    }
    with open(out_file(mode), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print("%s: %.1f MB per launch (%.4f x the weight bytes)"
          % (out_file(mode), hbm / 1e6, hbm / weight_bytes))


if __name__ == "__main__":
    main(sys.argv)
