"""Pins of the oracle's rotate-and-quantize packer (CPU only).

Hand-worked groups fix the scale rule and the rounding; exact grid values
must survive a round trip; after rotation every element is within half a
step of the fp64 rotated weight; the rotated product matches the unrotated
one within the quantization bound (which fixes the orientation W' = W H,
x' = H x); and on weights with outlier channels the rotation lowers the
error, the direction the fastgemma page reports.
"""
import numpy as np
import pytest

from bit_weight_only_w4a16_amd import synth


def _codes(oracle_mod, P, N, K):
    return oracle_mod.codes(P, N, K)


def test_hand_worked_group(oracle_mod):
    W = np.zeros((1, 32), dtype=np.float32)
    W[0, :8] = [7.0, 2.5, 3.5, -0.5, -1.5, 6.9, -7.0, 0.49]
    P, S = oracle_mod.quantize(W, 32, 0)
    assert S[0, 0] == 0x3F80                     # max 7 -> scale 1
    c = _codes(oracle_mod, P, 1, 32)[0]
    # 2.5 -> 2 and 3.5 -> 4 (ties to even), -0.5 -> -0 -> 0, 0.49 -> 0
    assert list(c[:8]) == [15, 10, 12, 8, 6, 15, 1, 8]
    assert np.all(c[8:] == 8)


def test_hand_worked_rounded_scale(oracle_mod):
    # max 1.0: 1/7 = 0x3E124925 in fp32 -> bf16 0x3E12 = 0.142578125
    W = np.zeros((1, 32), dtype=np.float32)
    W[0, :4] = [1.0, 0.5, -0.25, 0.0712890625]   # last = half a step exactly
    P, S = oracle_mod.quantize(W, 32, 0)
    assert S[0, 0] == 0x3E12
    c = _codes(oracle_mod, P, 1, 32)[0]
    # 1/0.142578125 = 7.0137 -> 7; 0.5/.. = 3.5068 -> 4; -0.25/.. = -1.7534 -> -2;
    # 0.0712890625/0.142578125 = 0.5 -> 0 (tie to even)
    assert list(c[:4]) == [15, 12, 6, 8]


def test_all_zero_group(oracle_mod):
    W = np.zeros((2, 64), dtype=np.float32)
    W[1, 40] = -3.0
    P, S = oracle_mod.quantize(W, 32, 0)
    assert S[0, 0] == 0 and S[0, 1] == 0 and S[1, 0] == 0
    c = _codes(oracle_mod, P, 2, 64)
    assert np.all(c[0] == 8) and np.all(c[1, :32] == 8)
    assert c[1, 40] == 1                          # -3 is the group max -> -7


@pytest.mark.parametrize("group", [32, 256, 512])
def test_grid_values_round_trip(oracle_mod, group):
    rng = np.random.default_rng(group)
    N, K = 5, 512
    codes = rng.integers(1, 16, (N, K))           # no code 0: |q| <= 7
    codes[:, ::group] = 15                        # each group reaches q = 7
    sbits = rng.integers(0x3C00, 0x4100, (N, K // group)).astype(np.uint16)
    s = (sbits.astype(np.uint32) << 16).view(np.float32)
    W = ((codes - 8) * np.repeat(s, group, axis=1)).astype(np.float32)
    P, S = oracle_mod.quantize(W, group, 0)
    assert np.array_equal(S, sbits)
    assert np.array_equal(_codes(oracle_mod, P, N, K), codes)


def test_rotated_within_half_step(oracle_mod):
    W = synth.outlier_weights(16, 1536, 3)
    P, S = oracle_mod.quantize(W, 256, 512)
    Wr = oracle_mod.fwht(W.astype(np.float64), 512)          # fp64 rotation
    D = oracle_mod.dequant(P, S, 16, 1536, 256)
    step = np.repeat(oracle_mod.bf16_to_f64(S), 256, axis=1)
    # half a step, plus the fp32 rotation error (10 stages of 2^-24 relative)
    slack = 12 * 2.0 ** -24 * np.abs(W).sum(axis=1, keepdims=True) / np.sqrt(512) * 8
    assert np.all(np.abs(D - Wr) <= 0.5 * step + slack)


def test_rotated_product_matches_unrotated(oracle_mod):
    N, K = 24, 1536
    W = synth.outlier_weights(N, K, 4)
    P, S = oracle_mod.quantize(W, 256, 512)
    rng = np.random.default_rng(5)
    x = rng.standard_normal(K)
    xr = oracle_mod.fwht(x, 512)
    D = oracle_mod.dequant(P, S, N, K, 256)
    y_q = D @ xr
    y = W.astype(np.float64) @ x
    step = np.repeat(oracle_mod.bf16_to_f64(S), 256, axis=1)
    bound = (0.5 * step + 1e-6) @ np.abs(xr)
    assert np.all(np.abs(y_q - y) <= bound)
    # the wrong orientation (x not rotated) is off by far more
    assert np.linalg.norm(D @ x - y) > 5 * np.linalg.norm(y_q - y)


def _rel_err(oracle_mod, W, group, block):
    N, K = W.shape
    P, S = oracle_mod.quantize(W, group, block)
    D = oracle_mod.dequant(P, S, N, K, group)
    if block:
        D = oracle_mod.fwht(D, block)        # H is its own inverse: W = W' H
    return np.linalg.norm(D - W) / np.linalg.norm(W)


@pytest.mark.parametrize("group", [256, 32])
def test_rotation_lowers_error_on_outlier_weights(oracle_mod, group):
    W = synth.outlier_weights(64, 1536, 11)
    plain = _rel_err(oracle_mod, W, group, 0)
    rot = _rel_err(oracle_mod, W, group, 512)
    assert rot < 0.7 * plain, (plain, rot)
    # without outliers the rotation changes little
    G = np.random.default_rng(12).standard_normal((64, 1536)).astype(np.float32)
    assert abs(_rel_err(oracle_mod, G, group, 512) - _rel_err(oracle_mod, G, group, 0)) < 0.03
