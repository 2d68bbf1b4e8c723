"""Pins of the oracle's decode attention (CPU only): closed forms (uniform
scores give the mean of the valid rows; a score gap of ln 3 gives weights 3/4
and 1/4; a dominant score returns that row), and invariants (slot order,
masked slots equal removed rows, the ring window, linearity in V)."""
import math

import numpy as np
import pytest


def _bf16(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _f(h):
    return (np.asarray(h, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def _rand(rng, shape):
    return _bf16(rng.standard_normal(shape).astype(np.float32))


def test_zero_query_is_mean_of_rows(oracle_mod):
    rng = np.random.default_rng(1)
    q = np.zeros((8, 256), np.uint16)
    K, V = _rand(rng, (37, 256)), _rand(rng, (37, 256))
    o, _ = oracle_mod.attn_decode(q, K, V, 0.125)
    assert np.allclose(o, np.broadcast_to(_f(V).mean(axis=0), o.shape), rtol=0, atol=1e-12)


def test_two_slots_weights_three_quarters(oracle_mod):
    rng = np.random.default_rng(2)
    D = 256
    q = np.zeros((8, D), np.uint16)
    q[:, 0] = 0x3F80                                   # 1.0
    K = np.zeros((2, D), np.uint16)
    K[0, 0] = 0x4000                                   # 2.0 -> score 2 * scale
    V = _rand(rng, (2, D))
    o, _ = oracle_mod.attn_decode(q, K, V, math.log(3.0) / 2.0)
    want = 0.75 * _f(V[0]) + 0.25 * _f(V[1])
    assert np.allclose(o, np.broadcast_to(want, o.shape), rtol=0, atol=1e-12)


def test_dominant_score_returns_row(oracle_mod):
    rng = np.random.default_rng(3)
    D = 512
    q = np.zeros((8, D), np.uint16)
    q[:, 3] = 0x3F80
    K = np.zeros((10, D), np.uint16)
    K[6, 3] = 0x4480                                   # 1024 -> exp(-1024 * 1) == 0
    V = _rand(rng, (10, D))
    o, _ = oracle_mod.attn_decode(q, K, V, 1.0)
    assert np.array_equal(o, np.broadcast_to(_f(V[6]), o.shape))


def test_slot_order_does_not_matter(oracle_mod):
    rng = np.random.default_rng(4)
    q, K, V = _rand(rng, (8, 256)), _rand(rng, (50, 256)), _rand(rng, (50, 256))
    perm = rng.permutation(50)
    o1, _ = oracle_mod.attn_decode(q, K, V, 0.0625)
    o2, _ = oracle_mod.attn_decode(q, K[perm], V[perm], 0.0625)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12)


def test_masked_slots_equal_removed_rows(oracle_mod):
    rng = np.random.default_rng(5)
    q, K, V = _rand(rng, (8, 256)), _rand(rng, (40, 256)), _rand(rng, (40, 256))
    pos = np.arange(40, dtype=np.int32)
    pos[[3, 17, 39]] = -1                              # empty slots
    keep = pos >= 0
    o1, _ = oracle_mod.attn_decode(q, K, V, 0.0625, pos=pos, cur=100)
    o2, _ = oracle_mod.attn_decode(q, K[keep], V[keep], 0.0625)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12)


def test_ring_window(oracle_mod):
    """A 16-slot ring written for positions 0..40 holds positions 25..40;
    window 10 at cur = 40 keeps positions 31..40."""
    rng = np.random.default_rng(6)
    D = 256
    q = _rand(rng, (8, D))
    Kf, Vf = _rand(rng, (41, D)), _rand(rng, (41, D))   # rows by position
    slots = 16
    pos = np.full(slots, -1, np.int32)
    K = np.zeros((slots, D), np.uint16)
    V = np.zeros((slots, D), np.uint16)
    for p in range(41):
        pos[p % slots] = p
        K[p % slots], V[p % slots] = Kf[p], Vf[p]
    o1, _ = oracle_mod.attn_decode(q, K, V, 0.0625, pos=pos, cur=40, window=10)
    o2, _ = oracle_mod.attn_decode(q, Kf[31:41], Vf[31:41], 0.0625)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12)


def test_linear_in_values(oracle_mod):
    rng = np.random.default_rng(7)
    q, K = _rand(rng, (8, 256)), _rand(rng, (30, 256))
    # V1 + V2 exact in bf16: small integers
    V1 = _bf16(rng.integers(-8, 8, (30, 256)).astype(np.float32))
    V2 = _bf16(rng.integers(-8, 8, (30, 256)).astype(np.float32))
    V12 = _bf16((_f(V1) + _f(V2)).astype(np.float32))
    o1, _ = oracle_mod.attn_decode(q, K, V1, 0.0625)
    o2, _ = oracle_mod.attn_decode(q, K, V2, 0.0625)
    o12, _ = oracle_mod.attn_decode(q, K, V12, 0.0625)
    assert np.allclose(o12, o1 + o2, rtol=1e-12, atol=1e-12)


def test_no_valid_slot_is_nan(oracle_mod):
    q = np.zeros((8, 256), np.uint16)
    K = np.zeros((4, 256), np.uint16)
    pos = np.array([-1, 50, 60, -1], np.int32)         # all in the future of cur = 10
    o, _ = oracle_mod.attn_decode(q, K, K, 1.0, pos=pos, cur=10)
    assert np.all(np.isnan(o))
