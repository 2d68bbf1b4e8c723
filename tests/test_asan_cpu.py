"""Host-side AddressSanitizer and UndefinedBehaviorSanitizer run, no GPU.

Builds the library's sources (device code as usual, host code instrumented)
with the driver tests/asan/driver.cpp and the oracle (oracle/oracle.c,
instrumented), then runs the driver: argument validation of every C-ABI
family before its first HIP call, the host packer and unpacker on ragged
shapes, the dispatcher's tile choice and text over many shapes and short
buffers, and every oracle routine on small inputs.  Any sanitizer report
aborts the driver; the test needs "ALL OK" and exit status 0.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_weight_only_w4a16_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")

# host-side instrumentation only: each -fsanitize= goes to the host pass
HOST_SAN = ["-Xarch_host", "-fsanitize=address",
            "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]
C_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
         "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(
    not all(os.path.exists(p) for p in (HIPCC, CLANG, CLANGXX)),
    reason="ROCm compilers not found")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("%s\n%s" % (" ".join(cmd), r.stderr[-4000:]))


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("asan"))
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    srcs.append(os.path.join(ROOT, "tests", "asan", "driver.cpp"))
    flags = ["-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include")] + HOST_SAN
    objs = [os.path.join(out, os.path.basename(s) + ".o") for s in srcs]
    jobs = max(1, min(8, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda so: _run([HIPCC] + flags + ["-c", so[0], "-o", so[1]], out),
                    zip(srcs, objs)))
    oracle_o = os.path.join(out, "oracle.o")
    _run([CLANG, "-O1", "-g"] + C_SAN + ["-c", os.path.join(ROOT, "oracle", "oracle.c"),
                                           "-o", oracle_o], out)
    exe = os.path.join(out, "driver")
    _run([CLANGXX] + C_SAN[:1] + ["-o", exe] + objs + [oracle_o,
          "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lm"], out)
    yield exe
    shutil.rmtree(out, ignore_errors=True)


def test_host_code_under_sanitizers(driver):
    env = dict(os.environ)
    # the HIP runtime's own allocations outlive main: leaks are not checked
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "ALL OK" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
