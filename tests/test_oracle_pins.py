"""Pins of the oracle to facts the pages and mathematics fix (CPU only).

Each test checks the oracle against something other than itself: a
hand-typed table, the pages' own float trick, a dense brute force built from
integer codes with numpy's matmul, exact invariants, or printed figures.
"""
import os
import struct

import numpy as np
import pytest

from bit_weight_only_w4a16_amd import accounting, synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _pack_from_codes(C):
    """Independent packer used only to build test inputs: codes (N, K) ints in
    0..15 -> canonical words, element 8w+j at bits [4j, 4j+4)."""
    C = np.asarray(C, dtype=np.uint64)
    N, K = C.shape
    C3 = C.reshape(N, K // 8, 8)
    words = np.zeros((N, K // 8), dtype=np.uint64)
    for j in range(8):
        words += C3[:, :, j] * np.uint64(16 ** j)
    return words.astype(np.uint32)


# ---------------------------------------------------------------- decode ---

def test_decode_table_hand_typed(oracle_mod):
    rows = _golden_rows("decode_words.txt")
    assert len(rows) >= 8
    one = np.array([[0x3F80]], dtype=np.uint16)   # bf16 1.0
    for row in rows:
        word = int(row[0], 16)
        expect = [int(v) for v in row[1:]]
        P = np.array([[word]], dtype=np.uint32)
        got = [oracle_mod.weight(P, one, 8, 8, 0, k) for k in range(8)]
        assert got == expect, (row[0], got, expect)
        codes = oracle_mod.codes(P, 1, 8)[0].tolist()
        assert [c - 8 for c in codes] == expect


def test_decode_matches_or_magic_trick(oracle_mod):
    """[P1] paragraph on the w4gemv.py kernel: OR the 4-bit value into the
    bits of 2^23 and subtract 2^23 + 8, exactly.  Checked for all 16 codes in
    every nibble position against the oracle's integer decode."""
    one = np.array([[0x3F80]], dtype=np.uint16)
    for c in range(16):
        trick = struct.unpack("<f", struct.pack("<I", 0x4B000000 | c))[0]
        trick = np.float32(trick) - np.float32(8388616.0)
        assert float(trick) == c - 8
        for j in range(8):
            P = np.array([[0x88888888 & ~(0xF << (4 * j)) | (c << (4 * j))]],
                         dtype=np.uint32)
            assert oracle_mod.weight(P, one, 8, 8, 0, j) == float(trick)
            # the other positions stay at code 8 -> exactly zero
            for jj in range(8):
                if jj != j:
                    assert oracle_mod.weight(P, one, 8, 8, 0, jj) == 0.0


def test_bf16_widening_exact(oracle_mod):
    h = np.array([0x3F80, 0xBF80, 0x4300, 0x0000, 0x8000, 0x3C00, 0x7F7F,
                  0x0001], dtype=np.uint16)
    expect = [1.0, -1.0, 128.0, 0.0, -0.0, 2.0 ** -7, 3.3895313892515355e38,
              2.0 ** -133]
    got = oracle_mod.bf16_to_f64(h)
    assert got.tolist() == expect


# ----------------------------------------------------------- brute force ---

@pytest.mark.parametrize("N", [1, 33, 65, 97])
@pytest.mark.parametrize("K,group", [(32, 32), (64, 32), (96, 32), (288, 32),
                                     (256, 256), (512, 256)])
@pytest.mark.parametrize("M", [1, 3])
def test_gemm_vs_dense_bruteforce(oracle_mod, N, K, group, M):
    rng = np.random.default_rng(1000 * N + K + M)
    C = rng.integers(0, 16, size=(N, K))
    P = _pack_from_codes(C)
    S = synth.f32_to_bf16_bits(
        np.abs(rng.standard_normal((N, K // group))).astype(np.float32) * 0.02 + 1e-3)
    X = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    s64 = synth.bf16_bits_to_f32(S).astype(np.float64)
    x64 = synth.bf16_bits_to_f32(X).astype(np.float64)
    W = (C.astype(np.float64) - 8.0) * np.repeat(s64, group, axis=1)
    # dequant is exact
    assert np.array_equal(oracle_mod.dequant(P, S, N, K, group), W)
    # product agrees with numpy's matmul to rounding
    Yref = np.matmul(x64, W.T)
    Y, A = oracle_mod.gemm(P, S, N, K, group, x64)
    Aref = np.matmul(np.abs(x64), np.abs(W).T)
    assert np.allclose(Y, Yref, rtol=0, atol=1e-12 * max(1.0, np.abs(Aref).max()))
    assert np.allclose(A, Aref, rtol=1e-13, atol=0)


def test_gemm_transposed_or_swapped_operands_would_fail(oracle_mod):
    """Guard the pin itself: a transposed weight or a wrong nibble order must
    change the result on a non-symmetric input."""
    rng = np.random.default_rng(7)
    N, K = 16, 64
    C = rng.integers(0, 16, size=(N, K))
    P = _pack_from_codes(C)
    S = np.full((N, K // 32), 0x3F80, dtype=np.uint16)
    x = rng.integers(-3, 4, size=K).astype(np.float64)
    Y, _ = oracle_mod.gemm(P, S, N, K, 32, x)
    assert np.array_equal(Y, (C - 8) @ x)
    # msb-first nibble order gives a different answer
    C_rev = C.reshape(N, K // 8, 8)[:, :, ::-1].reshape(N, K)
    assert not np.array_equal(Y, (C_rev - 8) @ x)
    # two's complement reading gives a different answer
    C_tc = np.where(C >= 8, C - 16, C)
    assert not np.array_equal(Y, C_tc @ x)


# ------------------------------------------------------------ invariants ---

def _dyadic_case(rng, N, K, group):
    C = rng.integers(0, 16, size=(N, K))
    P = _pack_from_codes(C)
    # scales that are small dyadic rationals (exact sums in fp64)
    sv = rng.integers(1, 64, size=(N, K // group)).astype(np.float32) / 64.0
    S = synth.f32_to_bf16_bits(sv)
    assert np.array_equal(synth.bf16_bits_to_f32(S), sv)
    return C, P, S


def test_all_code_8_gives_exact_zero(oracle_mod):
    N, K = 9, 96
    P = np.full((N, K // 8), 0x88888888, dtype=np.uint32)
    rng = np.random.default_rng(3)
    S = synth.f32_to_bf16_bits(rng.random((N, K // 32)).astype(np.float32))
    X = synth.f32_to_bf16_bits(rng.standard_normal((2, K)).astype(np.float32))
    Y, A = oracle_mod.gemm_bf16(P, S, N, K, 32, X)
    assert np.all(Y == 0.0) and np.all(A == 0.0)


def test_linearity_in_x_exact(oracle_mod):
    rng = np.random.default_rng(11)
    N, K = 21, 160
    _, P, S = _dyadic_case(rng, N, K, 32)
    x1 = rng.integers(-5, 6, size=K).astype(np.float64)
    x2 = rng.integers(-5, 6, size=K).astype(np.float64)
    y1, _ = oracle_mod.gemm(P, S, N, K, 32, x1)
    y2, _ = oracle_mod.gemm(P, S, N, K, 32, x2)
    y12, _ = oracle_mod.gemm(P, S, N, K, 32, 2 * x1 - 3 * x2)
    assert np.array_equal(y12, 2 * y1 - 3 * y2)


def test_doubling_one_group_scale_doubles_its_contribution(oracle_mod):
    rng = np.random.default_rng(12)
    N, K, group = 7, 192, 32
    _, P, S = _dyadic_case(rng, N, K, group)
    x = rng.integers(-4, 5, size=K).astype(np.float64)
    y0, _ = oracle_mod.gemm(P, S, N, K, group, x)
    g = 3
    mask = np.zeros(K)
    mask[g * group:(g + 1) * group] = 1.0
    contrib, _ = oracle_mod.gemm(P, S, N, K, group, x * mask)
    S2 = S.copy()
    S2[:, g] = synth.f32_to_bf16_bits(2 * synth.bf16_bits_to_f32(S[:, g]))
    y2, _ = oracle_mod.gemm(P, S2, N, K, group, x)
    assert np.array_equal(y2 - y0, contrib)
    assert np.any(contrib != 0)


def test_joint_group_permutation_invariance(oracle_mod):
    rng = np.random.default_rng(13)
    N, K, group = 11, 256, 32
    C, P, S = _dyadic_case(rng, N, K, group)
    x = rng.integers(-4, 5, size=K).astype(np.float64)
    y0, _ = oracle_mod.gemm(P, S, N, K, group, x)
    perm = rng.permutation(K // group)
    Cp = C.reshape(N, K // group, group)[:, perm, :].reshape(N, K)
    Sp = S[:, perm]
    xp = x.reshape(K // group, group)[perm].reshape(K)
    yp, _ = oracle_mod.gemm(_pack_from_codes(Cp), Sp, N, K, group, xp)
    assert np.array_equal(y0, yp)


def test_one_hot_returns_dequantized_weight(oracle_mod):
    case = synth.single_gemv_small()
    N, K = case.N, case.K
    W = oracle_mod.dequant(case.P, case.S, N, K, 32)
    for k in (0, 1, 7, 8, 31, 32, 255, 511):
        e = np.zeros(K)
        e[k] = 1.0
        y, _ = oracle_mod.gemm(case.P, case.S, N, K, 32, e)
        assert np.array_equal(y, W[:, k])


# ------------------------------------------------------------------ FWHT ---

def _sylvester(n):
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.kron(np.array([[1.0, 1.0], [1.0, -1.0]]), H)
    return H / np.sqrt(n)


def _popcount_form(n):
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    bits = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    return np.where(bits % 2 == 0, 1.0, -1.0) / np.sqrt(n)


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 64, 512])
def test_fwht_matches_sylvester_matrix_and_closed_form(oracle_mod, n):
    rng = np.random.default_rng(n)
    X = rng.standard_normal((3, n))
    H = _sylvester(n)
    got = oracle_mod.fwht(X, n)
    assert np.allclose(got, X @ H.T, rtol=0, atol=1e-12 * n)
    if n <= 64:
        assert np.allclose(H, _popcount_form(n), atol=1e-15)


def test_fwht_identities(oracle_mod):
    n = 512
    rng = np.random.default_rng(5)
    x = rng.standard_normal(n)
    hx = oracle_mod.fwht(x, n)
    # orthonormal: norm preserved, H H = I
    assert abs(np.linalg.norm(hx) - np.linalg.norm(x)) < 1e-12 * n
    assert np.allclose(oracle_mod.fwht(hx, n), x, atol=1e-12)
    # H e0 = n^-1/2 * ones
    e0 = np.zeros(n)
    e0[0] = 1.0
    assert np.allclose(oracle_mod.fwht(e0, n), np.full(n, n ** -0.5), atol=1e-15)
    # H e_j has one sign pattern: row j of the Sylvester matrix
    ej = np.zeros(n)
    ej[37] = 1.0
    assert np.allclose(oracle_mod.fwht(ej, n), _sylvester(n)[:, 37], atol=1e-15)


def test_fwht_blocks_are_independent_and_contiguous(oracle_mod):
    rng = np.random.default_rng(6)
    K, B = 1536, 512
    x = rng.standard_normal(K)
    y = oracle_mod.fwht(x, B)
    Hb = _sylvester(B)
    for b in range(K // B):
        assert np.allclose(y[b * B:(b + 1) * B], Hb @ x[b * B:(b + 1) * B],
                           atol=1e-11)
    x2 = x.copy()
    x2[1024:] += 1.0
    y2 = oracle_mod.fwht(x2, B)
    assert np.array_equal(y[:1024], y2[:1024])
    assert not np.allclose(y[1024:], y2[1024:])


def test_hadamard_rotation_identity(oracle_mod):
    """[P2] section "What is in the file": W' = W H^T with a runtime FWHT of
    the activation gives the same product, for orthogonal H.  Here the stored
    weights are W' and the equivalent unrotated W = W' H_blk."""
    rng = np.random.default_rng(8)
    N, K, group, B = 24, 1024, 256, 512
    P, S = synth.draw_weights(rng, N, K, group)
    X = synth.draw_activations(rng, 2, K, outlier_frac=0.01)
    x64 = oracle_mod.bf16_to_f64(X)
    Wp = oracle_mod.dequant(P, S, N, K, group)
    Hblk = np.kron(np.eye(K // B), _sylvester(B))
    y_rot, _ = oracle_mod.gemm(P, S, N, K, group, oracle_mod.fwht(x64, B))
    y_plain = x64 @ (Wp @ Hblk).T
    assert np.allclose(y_rot, y_plain, rtol=0, atol=1e-10)


# ------------------------------------------------------- byte accounting ---

def test_byte_accounting_reproduces_printed_figures():
    g = {r[0]: float(r[1]) for r in _golden_rows("byte_accounting.txt")}
    vocab, hidden = int(g["vocab"]), int(g["hidden"])
    layer_el = int(g["layer_elements"])
    # bytes = elements x (4 bits + 16 bits / 32) via the accounting function
    per_token = (accounting.weight_bytes(1, layer_el, 32)
                 + accounting.weight_bytes(vocab, hidden, 32))
    assert round(per_token / 2 ** 20, 1) == g["mib_per_token"]
    assert round(accounting.gbps(per_token, g["v5_ms_per_token"] * 1e-3), 1) == g["v5_gbps"]
    # both printed (ms, GB/s) pairs agree to the precision they are printed at
    for v, nd in (("v5", 2), ("v4", 1)):
        ms_implied = per_token / (g[v + "_gbps"] * 1e9) * 1e3
        assert round(ms_implied, nd) == g[v + "_ms_per_token"]
    ple = accounting.weight_bytes(vocab, int(g["ple_width"]), 32)
    assert round((per_token + ple) / 2 ** 20) == g["model_mib_4bit"]
    assert vocab * hidden * 2 / 2 ** 30 == g["embed_gib_16bit"]
    assert round(vocab * hidden / 1e6) == g["embed_params_millions"]


def test_sweep_bytes():
    total = sum(c_N * c_K // 2 + c_N * (c_K // 32) * 2
                for _, c_N, c_K in synth.LAYER_SHAPES) * synth.N_LAYERS
    total += accounting.weight_bytes(synth.VOCAB, synth.HIDDEN, 32)
    assert total == 923_222_016
