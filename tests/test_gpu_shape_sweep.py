"""A seeded sweep of w4a16_gemm shapes across every dispatch path (the GEMV,
the vector-ALU and matrix-core small-M kernels, the split-K kernel, the DMA
ring and the register-staged matrix-core kernel), each against the fp64
oracle, with and without the run-time transform.  The shapes are drawn from
a fixed seed so the run is reproducible; the kernel each one takes is named
in the test id's note and every path of the list is required to appear."""
import numpy as np
import pytest

import bit_weight_only_w4a16_amd as w4
from bit_weight_only_w4a16_amd import synth

from _util import assert_within, device, from_dev, note, to_dev_bf16, upload_packed

pytestmark = pytest.mark.gpu

# (M range, N range, K choices, groups): each class aims at one path
_CLASSES = [
    ("gemv", (1, 1), (64, 3000), (256, 512, 1024, 1536, 2048), (32, 256)),
    ("smallm", (2, 16), (32, 2000), (256, 512, 1536), (32, 256, 512)),
    ("smallm_valu", (2, 4), (32, 3000), (256, 512, 1536), (32,)),
    ("splitk", (2, 32), (6144, 7000), (512, 1024, 1536, 2048), (32, 256, 512)),
    ("ring", (33, 160), (64, 1200), (256, 512, 1536, 3072), (32, 256, 512)),
    ("regs", (17, 80), (16, 80), (16384, 20480), (256, 512)),
]


def _draw_shapes(seed=20261202, per_class=5):
    rng = np.random.default_rng(seed)
    out = []
    for name, (m0, m1), (n0, n1), ks, groups in _CLASSES:
        for _ in range(per_class):
            M = int(rng.integers(m0, m1 + 1))
            N = int(rng.integers(n0, n1 + 1))
            K = int(rng.choice(ks))
            g = int(rng.choice([gg for gg in groups if K % gg == 0]))
            had = int(rng.choice([0, 512])) if K % 512 == 0 and M > 1 else 0
            out.append((name, M, N, K, g, had))
    return out


SHAPES = _draw_shapes()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    device()
    w4.device_check()


def test_every_path_is_drawn():
    """The drawn shapes reach every kernel family of w4a16_gemm."""
    kinds = set()
    for _, M, N, K, g, _had in SHAPES:
        d = w4.describe_dispatch(M, N, K, g)
        if d.startswith("mfma"):
            kinds.add("ring" if "dma-ring" in d else "regs")
        elif d.startswith("smallm"):
            kinds.add("smallm_mfma" if d.startswith("smallm mfma") else "smallm_valu")
        else:
            kinds.add(d.split()[0])
    assert {"gemv", "smallm_valu", "smallm_mfma", "splitk", "ring", "regs"} <= kinds, kinds


@pytest.mark.parametrize("cls,M,N,K,g,had", SHAPES)
def test_gemm_shape_sweep(oracle_mod, cls, M, N, K, g, had):
    desc = w4.describe_dispatch(M, N, K, g)
    note("shape sweep [%s] M=%d N=%d K=%d g=%d had=%d -> %s" % (cls, M, N, K, g, had, desc))
    case = synth.make_case("sweep_%s" % cls, N, K, g, M, M * 7919 + N * 31 + K + g, "bf16",
                           outlier_frac=0.01)
    packed = upload_packed(case.P, case.S, N, K, g)
    X = to_dev_bf16(case.X)
    x64 = oracle_mod.bf16_to_f64(case.X)
    xr = oracle_mod.fwht(x64, had) if had else x64
    Yr, A = oracle_mod.gemm(case.P, case.S, N, K, g, xr, threads=16)
    for out_dtype in ("f32", "bf16"):
        Y = from_dev(w4.gemm(packed, N, K, g, X, had_block=had, out_dtype=out_dtype))
        assert_within(Y.reshape(M, N), Yr.reshape(M, N), A.reshape(M, N), out_dtype,
                      "[%s] %s %s" % (cls, desc, out_dtype))
