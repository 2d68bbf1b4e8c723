"""GPU parity of the split-K matrix-core kernel (w4a16_gemm at 2..32 rows,
8..32 at group 32, on matrices of 128 or more 48-row tiles, K a multiple of
512 up to 2048) against the fp64 oracle: one and two activation tiles of 16
rows (ragged M inside each), K of 1 to 4 blocks per wave, groups 32, 256 and
512, ragged N, strided activations, near-zero rows, code-8 columns and
run-to-run determinism; and the row counts around it going to the other
kernels."""
import numpy as np
import pytest

import bit_weight_only_w4a16_amd as w4
from bit_weight_only_w4a16_amd import synth

from _util import (assert_within, device, from_dev, note, set_dispatch_env, to_dev_bf16,
                   upload_packed)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    device()
    w4.device_check()


def _check(oracle_mod, case, M, N, K, g, what, had=0):
    desc = w4.describe_dispatch(M, N, K, g)
    assert desc.startswith("splitk"), desc
    packed = upload_packed(case.P, case.S, N, K, g)
    X = to_dev_bf16(case.X)
    x64 = oracle_mod.bf16_to_f64(case.X)
    xr = oracle_mod.fwht(x64, had) if had else x64
    Yr, A = oracle_mod.gemm(case.P, case.S, N, K, g, xr, threads=16)
    for out_dtype in ("f32", "bf16"):
        Y = from_dev(w4.gemm(packed, N, K, g, X, had_block=had, out_dtype=out_dtype))
        assert_within(Y, Yr, A, out_dtype, "%s %s" % (what, out_dtype))


@pytest.mark.parametrize("M,g", [(m, g) for g in (256, 512) for m in (2, 3, 8, 16, 17, 31, 32)] +
                         [(m, 32) for m in (8, 9, 16, 17, 31, 32)])
def test_splitk_gate_up_shape(oracle_mod, M, g):
    """The gate+up projection shape (N = 12288, K = 1536: three blocks per
    wave), every row count class."""
    N, K = 12288, 1536
    note("splitk M=%d N=%d K=%d g=%d" % (M, N, K, g))
    case = synth.make_case("splitk", N, K, g, M, 5 * M + g, "bf16", outlier_frac=0.01)
    _check(oracle_mod, case, M, N, K, g, "splitk M=%d g=%d" % (M, g))


@pytest.mark.parametrize("M,N,K,g", [(8, 6145, 512, 32), (30, 6145, 512, 256),
                                     (7, 6200, 1024, 512), (32, 6200, 1024, 32),
                                     (20, 7000, 2048, 256), (25, 6150, 2048, 32),
                                     (2, 6150, 2048, 512), (17, 6145, 512, 512)])
def test_splitk_ragged_shapes(oracle_mod, M, N, K, g):
    """One, two and four 128-K blocks per wave, ragged N (the last tile's
    rows past N read row N - 1 and are not stored) and ragged M."""
    note("splitk ragged M=%d N=%d K=%d g=%d" % (M, N, K, g))
    case = synth.make_case("splitkr", N, K, g, M, M + N + K + g, "bf16", outlier_frac=0.01)
    _check(oracle_mod, case, M, N, K, g, "splitk ragged M=%d N=%d K=%d g=%d" % (M, N, K, g))


@pytest.mark.parametrize("M", [8, 32])
def test_splitk_prefill_hadamard(oracle_mod, M):
    """The prefill workload at 8 and 32 rows (group 256, N = 12288, K = 1536,
    512-point run-time transform) runs on this kernel."""
    case = synth.prefill_g256(M)
    N, K, g = case.N, case.K, case.group
    note("splitk prefill M=%d" % M)
    _check(oracle_mod, case, M, N, K, g, "splitk prefill M=%d" % M, had=512)


@pytest.mark.parametrize("M,g", [(4, 256), (24, 32), (32, 512)])
def test_splitk_strided_activations(oracle_mod, M, g):
    """Activation rows with a stride beyond K (a view into a wider buffer)."""
    import torch
    N, K = 6200, 1536
    note("splitk strided M=%d g=%d" % (M, g))
    case = synth.make_case("splitks", N, K, g, M, 3 * M + g, "bf16")
    packed = upload_packed(case.P, case.S, N, K, g)
    big = torch.full((M, K + 40), float("nan"), dtype=torch.bfloat16, device=device())
    big[:, :K] = to_dev_bf16(case.X)
    Yr, A = oracle_mod.gemm(case.P, case.S, N, K, g, oracle_mod.bf16_to_f64(case.X), threads=16)
    Y = from_dev(w4.gemm(packed, N, K, g, big[:, :K], out_dtype="f32"))
    assert_within(Y, Yr, A, "f32", "splitk strided")


@pytest.mark.parametrize("M,g", [(8, 256), (32, 256), (20, 32), (2, 512)])
def test_splitk_near_zero_rows(oracle_mod, M, g):
    """Rows whose codes are almost all 8, small activations at the non-8
    positions: every product enters exactly."""
    N, K = 12288, 1536
    note("splitk near-zero M=%d g=%d" % (M, g))
    case = synth.sparse_case("splitk0", N, K, g, M, 11 * M + g, "f32")
    _check(oracle_mod, case, M, N, K, g, "splitk near-zero M=%d g=%d" % (M, g))


@pytest.mark.parametrize("g", [256, 32])
def test_splitk_code8_columns_exact_zero(g):
    """Columns whose codes are all 8 come out exactly zero."""
    M, N, K = 30, 6200, 1024
    rng = np.random.default_rng(6)
    P, S = synth.draw_weights(rng, N, K, g)
    P[5, :] = 0x88888888
    P[6199, :] = 0x88888888
    packed = upload_packed(P, S, N, K, g)
    assert w4.describe_dispatch(M, N, K, g).startswith("splitk")
    X = to_dev_bf16(synth.draw_activations(rng, M, K, outlier_frac=0.01))
    Y = from_dev(w4.gemm(packed, N, K, g, X, out_dtype="f32"))
    assert np.all(Y[:, 5] == 0.0) and np.all(Y[:, 6199] == 0.0)
    assert np.all(Y[:, 6] != 0.0)


@pytest.mark.parametrize("M,g", [(32, 256), (16, 32), (3, 512)])
def test_splitk_deterministic(M, g):
    """Run to run bitwise (the four slice sums are added in slice order)."""
    N, K = 12288, 1536
    case = synth.make_case("splitkd", N, K, g, M, 21 + M, "bf16")
    packed = upload_packed(case.P, case.S, N, K, g)
    X = to_dev_bf16(case.X)
    a = from_dev(w4.gemm(packed, N, K, g, X, out_dtype="f32"))
    for _ in range(2):
        b = from_dev(w4.gemm(packed, N, K, g, X, out_dtype="f32"))
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_splitk_force_path_off(oracle_mod, monkeypatch):
    """W4_FORCE_PATH=no_splitk sends the same shapes to the other kernels,
    whose results agree with the oracle too."""
    set_dispatch_env(monkeypatch, W4_FORCE_PATH="no_splitk")
    N, K, g = 12288, 1536, 256
    for M in (8, 32):
        assert not w4.describe_dispatch(M, N, K, g).startswith("splitk")
        case = synth.make_case("splitkoff", N, K, g, M, 40 + M, "bf16")
        packed = upload_packed(case.P, case.S, N, K, g)
        X = to_dev_bf16(case.X)
        Yr, A = oracle_mod.gemm(case.P, case.S, N, K, g, oracle_mod.bf16_to_f64(case.X),
                                threads=16)
        Y = from_dev(w4.gemm(packed, N, K, g, X, out_dtype="f32"))
        assert_within(Y, Yr, A, "f32", "no_splitk M=%d" % M)


@pytest.mark.parametrize("M,N,K,g,kernel", [(33, 12288, 1536, 256, "mfma"), (64, 12288, 1536, 256, "mfma"),
                                            (4, 12288, 1536, 32, "smallm"), (7, 12288, 1536, 32, "smallm"),
                                            (16, 2560, 1536, 256, "smallm"),
                                            (20, 12288, 3072, 256, "mfma")])
def test_splitk_boundaries(oracle_mod, M, N, K, g, kernel):
    """Just outside the split-K kernel's range (more than 32 rows, group 32
    below 8 rows, fewer than 128 workgroups, K beyond 2048) the other
    kernels take the product, and agree with the oracle."""
    desc = w4.describe_dispatch(M, N, K, g)
    assert desc.startswith(kernel), desc
    note("splitk boundary M=%d N=%d K=%d g=%d -> %s" % (M, N, K, g, desc))
    case = synth.make_case("splitkb", N, K, g, M, 7 * M + N + g, "bf16", outlier_frac=0.01)
    packed = upload_packed(case.P, case.S, N, K, g)
    X = to_dev_bf16(case.X)
    Yr, A = oracle_mod.gemm(case.P, case.S, N, K, g, oracle_mod.bf16_to_f64(case.X), threads=16)
    Y = from_dev(w4.gemm(packed, N, K, g, X, out_dtype="f32"))
    assert_within(Y, Yr, A, "f32", "boundary %s" % desc)
