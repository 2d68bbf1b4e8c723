"""GPU parity of split-K decode attention (8 query heads, 1 KV head)
against the fp64 oracle, full-length caches and position-tagged rings.

Acceptance: |gpu - oracle| <= 5e-3 * sum_t p_t |v_t| / sum_t p_t per output
(the softmax weights enter the value product as bf16: a relative error of at
most 2^-9 each, so at most 2^-8 of that scale, plus fp32 rounding).
"""
import math

import numpy as np
import pytest

import bit_weight_only_w4a16_amd as w4

from _util import device, note

pytestmark = pytest.mark.gpu


def _bf16(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).to(device())
    return t.view(torch.bfloat16) if a.dtype == np.uint16 else t


def _inputs(T, D, seed, peak=1.0):
    rng = np.random.default_rng(seed)
    q = _bf16(rng.standard_normal((8, D)) * peak)
    K = _bf16(rng.standard_normal((T, D)))
    V = _bf16(rng.standard_normal((T, D)))
    return q, K, V


def _run(q, K, V, T, scale, pos=None, cur=0, window=0, out_dtype="f32", poison=False):
    import torch
    Kd = _dev(K.view(np.int16)).view(torch.bfloat16)
    Vd = _dev(V.view(np.int16)).view(torch.bfloat16)
    Vt = w4.attn_pack_v(Vd, T)
    if poison:
        # slots past T in the last block hold NaN: the kernel must not use them
        D = K.shape[1]
        tail = ((T + 31) // 32) * 32
        if tail > T:
            blk = Vt.view(-1, D, 32)
            blk[-1, :, T % 32:] = float("nan")
    posd = None if pos is None else _dev(pos.astype(np.int32))
    out = w4.attn_decode(_dev(q.view(np.int16)).view(torch.bfloat16), Kd, Vt, T, scale,
                         pos=posd, cur=cur, window=window, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def _check(oracle_mod, got, q, K, V, scale, pos=None, cur=0, window=0, what=""):
    ref, absref = oracle_mod.attn_decode(q, K, V, scale, pos=pos, cur=cur, window=window)
    bound = 5e-3 * absref + 1e-30
    err = np.abs(got - ref)
    bad = ~(err <= bound)
    assert not bad.any(), "%s: %d bad, worst err/bound %.3g at %s" % (
        what, int(bad.sum()), float(np.nanmax(err / bound)), np.argwhere(bad)[0])
    return float(np.max(err / bound))


@pytest.mark.parametrize("D", [256, 512])
@pytest.mark.parametrize("T", [1, 5, 31, 32, 33, 100, 513, 4097, 20000])
def test_full_cache(oracle_mod, D, T):
    device()
    scale = 1.0 / math.sqrt(D)
    q, K, V = _inputs(T, D, 10 * T + D)
    note("attention full D=%d T=%d" % (D, T))
    got = _run(q, K, V, T, scale, poison=True)
    _check(oracle_mod, got, q, K, V, scale, what="D=%d T=%d" % (D, T))


@pytest.mark.parametrize("D,T", [(512, 131072), (256, 65536 + 7)])
def test_long_context(oracle_mod, D, T):
    """Several tiles per workgroup (the slice count saturates at 512)."""
    device()
    scale = 1.0 / math.sqrt(D)
    q, K, V = _inputs(T, D, 77 + D)
    note("attention long D=%d T=%d" % (D, T))
    got = _run(q, K, V, T, scale)
    _check(oracle_mod, got, q, K, V, scale, what="long D=%d T=%d" % (D, T))


@pytest.mark.parametrize("peak", [4.0, 16.0])
def test_peaky_scores(oracle_mod, peak):
    """Large scores: the softmax is dominated by a few slots."""
    device()
    D, T = 512, 3000
    q, K, V = _inputs(T, D, 5, peak=peak)
    got = _run(q, K, V, T, 1.0 / math.sqrt(D))
    _check(oracle_mod, got, q, K, V, 1.0 / math.sqrt(D), what="peak %g" % peak)


@pytest.mark.parametrize("window", [512, 300, 0])
def test_ring(oracle_mod, window):
    """A 512-slot ring written for positions 0..1300 (wrapped), some slots
    empty, never-written slots holding NaN; window 512 / 300 / none."""
    import torch
    device()
    D, S, cur = 256, 512, 1300
    rng = np.random.default_rng(window + 3)
    q = _bf16(rng.standard_normal((8, D)))
    K = _bf16(rng.standard_normal((S, D)))
    V = _bf16(rng.standard_normal((S, D)))
    pos = np.array([cur - ((cur - s) % S) for s in range(S)], dtype=np.int32)
    pos[[7, 100, 300]] = -1
    K[[7, 100, 300]] = 0x7FC0                          # NaN keys in empty slots
    V[[7, 100, 300]] = 0x7FC0
    got = _run(q, K, V, S, 0.0625, pos=pos, cur=cur, window=window)
    _check(oracle_mod, got, q, K, V, 0.0625, pos=pos, cur=cur, window=window,
           what="ring window %d" % window)


def test_bf16_output_and_determinism(oracle_mod):
    device()
    D, T = 512, 777
    q, K, V = _inputs(T, D, 21)
    a = _run(q, K, V, T, 0.05, out_dtype="bf16")
    b = _run(q, K, V, T, 0.05, out_dtype="bf16")
    assert np.array_equal(a, b)
    ref, absref = oracle_mod.attn_decode(q, K, V, 0.05)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert np.all(np.abs(a - ref) <= 5e-3 * absref + ulp)


def test_no_valid_slot_gives_nan(oracle_mod):
    device()
    D, T = 256, 64
    q, K, V = _inputs(T, D, 2)
    pos = np.full(T, -1, np.int32)
    got = _run(q, K, V, T, 0.1, pos=pos, cur=5)
    assert np.all(np.isnan(got))


def test_store_kv_then_attend(oracle_mod):
    """Decode-step cache writes slot by slot give the same result as packing."""
    import torch
    device()
    D, T = 512, 70
    q, K, V = _inputs(T, D, 8)
    Kd = torch.zeros((96, D), dtype=torch.bfloat16, device=device())
    Vt = torch.zeros(96 * D, dtype=torch.bfloat16, device=device())
    Kh = _dev(K.view(np.int16)).view(torch.bfloat16)
    Vh = _dev(V.view(np.int16)).view(torch.bfloat16)
    for t in range(T):
        w4.attn_store_kv(Kh[t], Vh[t], t, Kd, Vt)
    out = w4.attn_decode(_dev(q.view(np.int16)).view(torch.bfloat16), Kd, Vt, T, 0.05)
    torch.cuda.synchronize()
    _check(oracle_mod, out.cpu().numpy().astype(np.float64), q, K, V, 0.05, what="store_kv")
