"""GPU parity of the blockwise FWHT (w4_fwht), the small-M product
(w4a16_gemm_smallM) and the prefill entry point (w4a16_gemm) against the fp64
oracle.  The prefill workload is group 256, N=12288, K=1536 with a 512-point
Hadamard rotation along K and activations with 1% outliers x20."""
import numpy as np
import pytest

import bit_weight_only_w4a16_amd as w4
from bit_weight_only_w4a16_amd import synth

from _util import (assert_within, bf16_ulp, device, from_dev, note, set_dispatch_env,
                   to_dev_bf16, upload_packed)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    device()
    w4.device_check()


# ------------------------------------------------------------------ FWHT ---

@pytest.mark.parametrize("M,K,block", [(8, 1536, 512), (64, 1536, 512), (512, 1536, 512),
                                       (3, 1024, 1024), (5, 256, 2), (7, 96, 32),
                                       (2, 512, 64), (9, 384, 128), (1, 4096, 256)])
def test_fwht_vs_oracle(oracle_mod, M, K, block):
    note("fwht M=%d K=%d block=%d" % (M, K, block))
    rng = np.random.default_rng(M * K + block)
    Xb = synth.draw_activations(rng, M, K, outlier_frac=0.01)
    X = to_dev_bf16(Xb)
    got = from_dev(w4.fwht(X, block)).astype(np.float64)
    ref = oracle_mod.fwht(oracle_mod.bf16_to_f64(Xb), block)
    # bf16 rounding of the fp32 result (half an ulp) plus fp32 butterfly error
    absx = np.abs(oracle_mod.bf16_to_f64(Xb)).reshape(M, K // block, block).sum(-1)
    fp32_err = np.repeat(absx, block, axis=1) * (np.log2(block) + 2) * 2.0 ** -24
    err = np.abs(got - ref)
    assert np.all(err <= 0.5 * bf16_ulp(ref) * 1.0001 + fp32_err + 1e-30), err.max()


def test_fwht_in_place_and_strided(oracle_mod):
    import torch
    M, K, block = 6, 1536, 512
    rng = np.random.default_rng(2)
    Xb = synth.draw_activations(rng, M, K)
    big = torch.zeros((M, K + 64), dtype=torch.bfloat16, device=device())
    big[:, :K] = to_dev_bf16(Xb)
    view = big[:, :K]
    ref = from_dev(w4.fwht(to_dev_bf16(Xb), block))
    w4.fwht(view, block, out=view)
    assert np.array_equal(from_dev(view), ref)
    assert np.all(from_dev(big[:, K:]) == 0.0)


def test_fwht_twice_is_identity_within_rounding():
    """H is symmetric and orthonormal, so applying the transform twice returns
    x up to the two roundings: the first rounding errors e_j (at most half an
    ulp of x'_j) pass through H (|(He)_i| <= sum_j |e_j| / sqrt(B)), then the
    second result is rounded (half an ulp)."""
    M, K, block = 4, 1536, 512
    rng = np.random.default_rng(9)
    Xb = synth.draw_activations(rng, M, K)
    X = to_dev_bf16(Xb)
    X1 = w4.fwht(X, block)
    back = from_dev(w4.fwht(X1, block)).astype(np.float64)
    x = synth.bf16_bits_to_f32(Xb).astype(np.float64)
    half_ulp_1 = 0.5 * bf16_ulp(from_dev(X1)).reshape(M, K // block, block).sum(-1)
    prop = np.repeat(half_ulp_1, block, axis=1) / np.sqrt(block)
    b = prop * 1.01 + 0.5 * bf16_ulp(np.abs(x) + prop) * 1.01 + 1e-6
    assert np.all(np.abs(back - x) <= b), float(np.max(np.abs(back - x) / b))


# --------------------------------------------------------------- small M ---

@pytest.mark.parametrize("M", [2, 3, 4, 5, 8, 11, 16])
@pytest.mark.parametrize("N,K,g", [(12288, 1536, 256), (97, 288, 32), (1536, 6144, 32),
                                   (33, 16384, 32), (65, 1024, 256), (129, 1536, 512),
                                   (12288, 1536, 32), (1000, 2048, 32), (2560, 1536, 32)])
def test_smallm_vs_oracle(oracle_mod, M, N, K, g):
    note("smallM M=%d N=%d K=%d g=%d" % (M, N, K, g))
    case = synth.make_case("smallm", N, K, g, M, 10 * M + N + K, "bf16")
    packed = upload_packed(case.P, case.S, N, K, g)
    X = to_dev_bf16(case.X)
    for out_dtype in ("bf16", "f32"):
        Y = from_dev(w4.gemm_smallM(packed, N, K, g, X, out_dtype))
        Yr, A = oracle_mod.gemm_bf16(case.P, case.S, N, K, g, case.X, threads=16)
        assert_within(Y, Yr, A, out_dtype, "smallM M=%d" % M)


@pytest.mark.parametrize("M,N,g", [(5, 3, 256), (3, 5, 32)])
def test_smallm_largest_k(oracle_mod, M, N, g):
    """Small M at the largest K the call accepts (2^20)."""
    K = 1 << 20
    note("smallM M=%d N=%d K=%d g=%d" % (M, N, K, g))
    case = synth.make_case("smk", N, K, g, M, 91 + M, "bf16")
    packed = upload_packed(case.P, case.S, N, K, g)
    X = to_dev_bf16(case.X)
    Yr, A = oracle_mod.gemm(case.P, case.S, N, K, g, oracle_mod.bf16_to_f64(case.X), threads=16)
    for out_dtype in ("bf16", "f32"):
        Y = from_dev(w4.gemm_smallM(packed, N, K, g, X, out_dtype=out_dtype))
        assert_within(Y, Yr, A, out_dtype, "smallM largest K %s" % out_dtype)


@pytest.mark.parametrize("M", [2, 8, 16])
@pytest.mark.parametrize("N,K,g", [(12288, 1536, 256), (129, 1536, 512), (12288, 1536, 32)])
def test_smallm_vector_alu_path(oracle_mod, monkeypatch, M, N, K, g):
    """The vector-ALU small-M kernels on shapes the matrix-core small-M
    kernel otherwise takes (W4_FORCE_PATH=smallm_valu keeps them)."""
    set_dispatch_env(monkeypatch, W4_FORCE_PATH="smallm_valu")
    note("smallM vector ALU M=%d N=%d K=%d g=%d" % (M, N, K, g))
    assert not w4.describe_dispatch(M, N, K, g).startswith("smallm mfma") or M > 8
    case = synth.make_case("smallv", N, K, g, M, 7 * M + N + K, "bf16")
    packed = upload_packed(case.P, case.S, N, K, g)
    X = to_dev_bf16(case.X)
    Y = from_dev(w4.gemm_smallM(packed, N, K, g, X, "f32"))
    Yr, A = oracle_mod.gemm_bf16(case.P, case.S, N, K, g, case.X, threads=16)
    assert_within(Y, Yr, A, "f32", "smallM VALU M=%d" % M)


@pytest.mark.parametrize("M", [2, 3, 4, 8, 16])
def test_smallm_fused_transform_bitwise(M):
    """With had_block = 512 the transform runs inside the matrix-core small-M
    kernel (up to 4 rows) or in the transform kernel before it (more rows):
    both bitwise equal to the transform kernel followed by the small-M
    product."""
    N, K, g = 1000, 1536, 256
    assert w4.describe_dispatch(M, N, K, g).startswith("smallm mfma")
    rng = np.random.default_rng(40 + M)
    P, S = synth.draw_weights(rng, N, K, g)
    packed = upload_packed(P, S, N, K, g)
    X = to_dev_bf16(synth.draw_activations(rng, M, K, outlier_frac=0.01))
    note("fused transform small-M M=%d" % M)
    Yf = from_dev(w4.gemm(packed, N, K, g, X, had_block=512, out_dtype="f32"))
    Ys = from_dev(w4.gemm_smallM(packed, N, K, g, w4.fwht(X, 512), "f32"))
    assert np.array_equal(Yf, Ys)


@pytest.mark.parametrize("g", [256, 32])
def test_smallm_mfma_code8_columns_exact_zero(g):
    """Columns whose codes are all 8 are exactly zero through the matrix-core
    small-M kernel (the offset chain goes through the same arithmetic)."""
    M, N, K = 8, 200, 1536
    assert w4.describe_dispatch(M, N, K, g).startswith("smallm mfma")
    rng = np.random.default_rng(6)
    P, S = synth.draw_weights(rng, N, K, g)
    P[3, :] = 0x88888888
    P[150, :] = 0x88888888
    packed = upload_packed(P, S, N, K, g)
    X = to_dev_bf16(synth.draw_activations(rng, M, K, outlier_frac=0.01))
    Y = from_dev(w4.gemm_smallM(packed, N, K, g, X, "f32"))
    assert np.all(Y[:, 3] == 0.0) and np.all(Y[:, 150] == 0.0)
    assert np.all(Y[:, 4] != 0.0)


@pytest.mark.parametrize("K", [1536, 288])
def test_smallm_rows_equal_gemv_bitwise(K):
    """Row m of the small-M product depends on X[m] only, bit for bit (the
    matrix-core kernel at K = 1536, the vector-ALU kernel at K = 288)."""
    import torch
    N, g, M = 2560, 32, 5
    case = synth.make_case("rows", N, K, g, M, 77, "f32")
    packed = upload_packed(case.P, case.S, N, K, g)
    X = to_dev_bf16(case.X)
    Y = from_dev(w4.gemm_smallM(packed, N, K, g, X, "f32"))
    X2 = X.clone()
    X2[3] = 0
    Y2 = from_dev(w4.gemm_smallM(packed, N, K, g, X2, "f32"))
    assert np.array_equal(Y[[0, 1, 2, 4]], Y2[[0, 1, 2, 4]])
    assert np.all(Y2[3] == 0.0)
    del torch


# ---------------------------------------------------- prefill (group 256) ---

@pytest.mark.parametrize("M", [8, 64, 512])
def test_prefill_g256_hadamard(oracle_mod, M):
    """The prefill workload: W' stored (drawn directly as the rotated weights),
    x' = FWHT_512(x) at run time.  The oracle uses the exact fp64 transform;
    the GPU rounds x' to bf16 before the product (within the tolerance)."""
    case = synth.prefill_g256(M)
    N, K, g = case.N, case.K, case.group
    note("prefill M=%d N=%d K=%d g=%d" % (M, N, K, g))
    packed = upload_packed(case.P, case.S, N, K, g)
    X = to_dev_bf16(case.X)
    try:
        Y = from_dev(w4.gemm(packed, N, K, g, X, had_block=512, out_dtype="bf16"))
    except w4.W4Error as e:
        if e.status == -5:
            pytest.skip("matrix-core tile not built: %s" % e)
        raise
    # every row, also at 512 (9.7 G multiply-adds: a few seconds of the
    # oracle on 16 threads)
    xr = oracle_mod.fwht(oracle_mod.bf16_to_f64(case.X), 512)
    Yr, A = oracle_mod.gemm(case.P, case.S, N, K, g, xr, threads=16)
    assert_within(Y, Yr, A, "bf16", "prefill M=%d" % M)


@pytest.mark.parametrize("M,N,K,g,had", [(17, 100, 256, 32, 0), (64, 12288, 1536, 32, 0),
                                         (100, 513, 1536, 256, 512), (512, 300, 512, 256, 0),
                                         (65, 1000, 2048, 256, 256), (33, 64, 256, 256, 0),
                                         (64, 12288, 1536, 512, 512), (40, 300, 1024, 512, 0),
                                         (9, 200, 512, 256, 0), (16, 1000, 1536, 32, 0),
                                         (13, 12288, 1536, 256, 512),
                                         # the largest K the call accepts (2^20)
                                         (20, 40, 1 << 20, 256, 0), (70, 24, 1 << 20, 32, 0)])
def test_matrix_core_gemm_shapes(oracle_mod, M, N, K, g, had):
    """M >= 9 runs on the matrix cores: ragged M and N, all group sizes, with
    and without the run-time transform, up to the largest K."""
    note("mfma gemm M=%d N=%d K=%d g=%d had=%d" % (M, N, K, g, had))
    case = synth.make_case("mfma", N, K, g, M, M * 31 + N + K, "bf16", outlier_frac=0.01)
    packed = upload_packed(case.P, case.S, N, K, g)
    X = to_dev_bf16(case.X)
    x64 = oracle_mod.bf16_to_f64(case.X)
    xr = oracle_mod.fwht(x64, had) if had else x64
    rows = np.arange(M) if M <= 128 else np.random.default_rng(1).choice(M, 64, replace=False)
    Yr, A = oracle_mod.gemm(case.P, case.S, N, K, g, xr[rows], threads=16)
    for out_dtype in ("bf16", "f32"):
        Y = from_dev(w4.gemm(packed, N, K, g, X, had_block=had, out_dtype=out_dtype))
        assert_within(Y[rows], Yr, A, out_dtype, "mfma %s" % out_dtype)


def test_matrix_core_largest_m(oracle_mod):
    """The largest M the call accepts (2^20 rows, 16384 row blocks), checked
    on sampled rows."""
    M, N, K, g = 1 << 20, 40, 256, 256
    note("mfma gemm largest M=%d N=%d K=%d g=%d" % (M, N, K, g))
    rng = np.random.default_rng(2024)
    P, S = synth.draw_weights(rng, N, K, g)
    X = synth.draw_activations(rng, M, K)
    packed = upload_packed(P, S, N, K, g)
    Xd = to_dev_bf16(X)
    rows = np.concatenate([[0, M - 1], rng.choice(M, 62, replace=False)])
    Yr, A = oracle_mod.gemm(P, S, N, K, g, oracle_mod.bf16_to_f64(X[rows]), threads=16)
    Y = from_dev(w4.gemm(packed, N, K, g, Xd, out_dtype="bf16"))
    assert_within(Y[rows], Yr, A, "bf16", "largest M")


@pytest.mark.parametrize("env,g", [({"W4_PREFILL_CFG": str(c)}, 256) for c in range(11)] +
                         [({"W4_PREFILL_CFG": str(c)}, 32) for c in range(11)] +
                         [({"W4_FORCE_PATH": "prefill_regs"}, 32)] +
                         [({"W4_PREFILL_CFG": "4"}, 512), ({"W4_PREFILL_CFG": "5"}, 512),
                          ({"W4_FORCE_PATH": "prefill_regs"}, 256), ({"W4_PREFILL_CFG": "7"}, 512)])
def test_matrix_core_every_tiling(oracle_mod, monkeypatch, env, g):
    """Every compiled matrix-core tiling (the tuning overrides select them,
    one per call) against the oracle on one ragged case; at group 512 the
    two-way K split falls back to an unsplit tiling (3 groups)."""
    set_dispatch_env(monkeypatch, **env)
    M, N, K = 70, 1000, 1536
    note("mfma tiling %s M=%d N=%d K=%d g=%d" % (env, M, N, K, g))
    case = synth.make_case("tile", N, K, g, M, 77, "bf16", outlier_frac=0.01)
    packed = upload_packed(case.P, case.S, N, K, g)
    X = to_dev_bf16(case.X)
    Yr, A = oracle_mod.gemm(case.P, case.S, N, K, g, oracle_mod.bf16_to_f64(case.X), threads=16)
    Y = from_dev(w4.gemm(packed, N, K, g, X, out_dtype="f32"))
    assert_within(Y, Yr, A, "f32", "tiling %s" % env)


@pytest.mark.parametrize("cfg,K,g", [(c, 6144, 256) for c in (0, 1, 4, 5, 6, 7, 8)] +
                         [(0, 8192, 256), (5, 8192, 256), (4, 8192, 256), (6, 6144, 512),
                          (7, 8192, 256), (7, 6144, 512), (9, 6144, 256), (9, 8192, 256),
                          (9, 6144, 512), (10, 8192, 256), (10, 1536, 32),
                          (5, 6144, 32), (1, 6144, 32), (4, 6144, 32), (0, 2048, 32)])
def test_matrix_core_many_scale_groups(oracle_mod, monkeypatch, cfg, K, g):
    """The DMA-ring tilings with 12 to 32 scale groups per row at groups 256
    and 512 (the down-projection K = 6144; K = 8192, the most the ring takes)
    and 64 to 192 at group 32 (only the split tilings hold more than 48; the
    others are replaced by the two-way split), ragged M and N; a split that
    does not divide the groups falls back unsplit."""
    set_dispatch_env(monkeypatch, W4_PREFILL_CFG=str(cfg))
    M, N = 70, 1000
    assert "dma-ring" in w4.describe_dispatch(M, N, K, g)
    note("mfma many groups cfg=%d M=%d N=%d K=%d g=%d" % (cfg, M, N, K, g))
    case = synth.make_case("groups", N, K, g, M, 91 + cfg, "bf16", outlier_frac=0.01)
    packed = upload_packed(case.P, case.S, N, K, g)
    X = to_dev_bf16(case.X)
    Yr, A = oracle_mod.gemm(case.P, case.S, N, K, g, oracle_mod.bf16_to_f64(case.X), threads=16)
    Y = from_dev(w4.gemm(packed, N, K, g, X, out_dtype="f32"))
    assert_within(Y, Yr, A, "f32", "cfg %d K %d g %d" % (cfg, K, g))


@pytest.mark.parametrize("M,g,slots", [(320, 256, "slots 4"), (321, 256, "slots 3"),
                                       (640, 256, "slots 4"), (641, 256, "slots 3"),
                                       (320, 32, "slots 4"), (321, 32, "slots 3")])
def test_ring_block_shape_boundaries(oracle_mod, M, g, slots):
    """Row counts on both sides of a block-shape change at N = 12288,
    K = 1536 (64 x 128 blocks, two workgroups per CU on a four-slot ring or
    three on a three-slot ring), on sampled rows including the last."""
    N, K = 12288, 1536
    desc = w4.describe_dispatch(M, N, K, g)
    assert "block 64x128" in desc and slots in desc, desc
    note("ring boundary M=%d g=%d -> %s" % (M, g, desc))
    rng = np.random.default_rng(M + g)
    P, S = synth.draw_weights(rng, N, K, g)
    X = synth.draw_activations(rng, M, K, outlier_frac=0.01)
    packed = upload_packed(P, S, N, K, g)
    rows = np.concatenate([[0, M - 1], rng.choice(M, 14, replace=False)])
    Yr, A = oracle_mod.gemm(P, S, N, K, g, oracle_mod.bf16_to_f64(X[rows]), threads=16)
    Y = from_dev(w4.gemm(packed, N, K, g, to_dev_bf16(X), out_dtype="bf16"))
    assert_within(Y[rows], Yr, A, "bf16", "boundary M=%d g=%d" % (M, g))


@pytest.mark.parametrize("cfg,K,g", [(c, K, g) for c in (9, 10) for K, g in ((256, 256), (512, 512),
                                                                          (512, 256))] +
                         [(10, 256, 32), (10, 512, 32)])
def test_matrix_core_short_k(oracle_mod, monkeypatch, cfg, K, g):
    """The three-slot and shared-decode tilings at their shortest K (four
    and eight 64-wide stages: the ring never wraps, or wraps twice), one
    and two scale groups, ragged M and N, against the oracle."""
    set_dispatch_env(monkeypatch, W4_PREFILL_CFG=str(cfg))
    M, N = 133, 1100
    assert "dma-ring" in w4.describe_dispatch(M, N, K, g)
    note("mfma short K cfg=%d M=%d N=%d K=%d g=%d" % (cfg, M, N, K, g))
    case = synth.make_case("shortk", N, K, g, M, 300 + cfg + K + g, "bf16", outlier_frac=0.01)
    packed = upload_packed(case.P, case.S, N, K, g)
    X = to_dev_bf16(case.X)
    Yr, A = oracle_mod.gemm(case.P, case.S, N, K, g, oracle_mod.bf16_to_f64(case.X), threads=16)
    for out_dtype in ("f32", "bf16"):
        Y = from_dev(w4.gemm(packed, N, K, g, X, out_dtype=out_dtype))
        assert_within(Y, Yr, A, out_dtype, "short K cfg %d K %d g %d" % (cfg, K, g))


@pytest.mark.parametrize("M,N,K,g", [(512, 12288, 1536, 256), (300, 1000, 1536, 512),
                                     (129, 12288, 256, 256), (1024, 1536, 6144, 256)])
def test_shared_decode_matches_per_wave_decode_bitwise(monkeypatch, M, N, K, g):
    """The shared-decode tiling forms the same products in the same order as
    the per-wave-decode tiling (same K permutation, groups accumulated from
    zero and scaled into the totals in group order): their outputs agree bit
    for bit, in fp32 and bf16, including ragged blocks and a K of four stages."""
    rng = np.random.default_rng(M + N + K)
    P, S = synth.draw_weights(rng, N, K, g)
    packed = upload_packed(P, S, N, K, g)
    X = to_dev_bf16(synth.draw_activations(rng, M, K, outlier_frac=0.01))
    note("shared decode bitwise M=%d N=%d K=%d g=%d" % (M, N, K, g))
    for out_dtype in ("f32", "bf16"):
        outs = []
        for cfg in ("0", "9"):
            set_dispatch_env(monkeypatch, W4_PREFILL_CFG=cfg)
            d = w4.describe_dispatch(M, N, K, g)
            assert ("shared-decode" in d) == (cfg == "9"), d
            outs.append(from_dev(w4.gemm(packed, N, K, g, X, out_dtype=out_dtype)))
        assert np.array_equal(outs[0].view(np.uint8), outs[1].view(np.uint8)), out_dtype


@pytest.mark.parametrize("g", [256, 32])
def test_matrix_core_code8_columns_exact_zero(g):
    """Columns whose codes are all 8 are exactly zero through the matrix-core
    path (every operand is the exact (c - 8), so such a column's products are
    all exact zeros)."""
    M, N, K = 64, 128, 1536
    rng = np.random.default_rng(4)
    P, S = synth.draw_weights(rng, N, K, g)
    P[5, :] = 0x88888888
    P[77, :] = 0x88888888
    packed = upload_packed(P, S, N, K, g)
    X = to_dev_bf16(synth.draw_activations(rng, M, K, outlier_frac=0.01))
    Y = from_dev(w4.gemm(packed, N, K, g, X, out_dtype="f32"))
    assert np.all(Y[:, 5] == 0.0) and np.all(Y[:, 77] == 0.0)
    assert np.all(Y[:, 6] != 0.0)


@pytest.mark.parametrize("M,had,g,K", [(512, 0, 256, 1536), (200, 0, 256, 1536),
                                       (64, 0, 256, 1536), (16, 512, 256, 1536),
                                       (8, 0, 256, 1536), (3, 512, 256, 1536),
                                       (512, 0, 32, 1536), (64, 0, 32, 1536),
                                       (64, 0, 32, 6144)])
def test_matrix_core_deterministic(M, had, g, K):
    """Run to run bitwise: the tiled matrix-core kernels (512, 200 and 64 rows,
    K-split workgroups included, groups 256 and 32) and the matrix-core
    small-M kernel (with and without the fused transform)."""
    N = 1024
    case = synth.make_case("det", N, K, g, M, 9 + M, "bf16")
    packed = upload_packed(case.P, case.S, N, K, g)
    X = to_dev_bf16(case.X)
    a = from_dev(w4.gemm(packed, N, K, g, X, had_block=had, out_dtype="f32"))
    for _ in range(2):
        b = from_dev(w4.gemm(packed, N, K, g, X, had_block=had, out_dtype="f32"))
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
