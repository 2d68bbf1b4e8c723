"""GPU parity of the int8 twin: the per-row int8 quantizer bit for bit
against the oracle; the int8 matrix-core GEMM against the exact integer
product (three fp32 roundings: the int32 -> fp32 conversion and two scale
multiplications); and the auto:M switch (int4 below switch_rows, int8 twin at
or above) end to end."""
import numpy as np
import pytest

import bit_weight_only_w4a16_amd as w4
from bit_weight_only_w4a16_amd import synth

from _util import device, note, to_dev_bf16, upload_packed, set_dispatch_env

pytestmark = pytest.mark.gpu

REL = 4 * 2.0 ** -24


def _t(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device())


def _bf16_bits(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("N,K,blk", [(33, 512, 0), (100, 1536, 512), (12288, 1536, 512),
                                     (7, 6144, 512), (5, 8, 0), (64, 2048, 64), (300, 1536, 256)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_rows_bit_exact(oracle_mod, N, K, blk, dtype):
    import torch
    device()
    W = synth.outlier_weights(N, K, N + K + blk)
    W[0] = 0.0                                   # a zero row
    if dtype == "bf16":
        Wt = _t(W).to(torch.bfloat16)
        W = Wt.float().cpu().numpy()
    else:
        Wt = _t(W)
    note("int8 quantize N=%d K=%d block=%d %s" % (N, K, blk, dtype))
    Q, S = w4.quantize_rows_i8(Wt, blk)
    torch.cuda.synchronize()
    Qo, So = oracle_mod.quantize_rows_i8(W, blk)
    assert np.array_equal(S.cpu().numpy().view(np.uint32), So.view(np.uint32))
    bad = np.argwhere(Q.cpu().numpy() != Qo)
    assert bad.size == 0, (tuple(bad[0]),)


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (17, 100, 256), (64, 12288, 1536),
                                   (512, 12288, 1536), (33, 1000, 2048), (130, 64, 6144),
                                   (200, 513, 128)])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_gemm_i8_vs_exact(oracle_mod, M, N, K, out_dtype):
    import torch
    device()
    rng = np.random.default_rng(M + N + K)
    Xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    Wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    xs = (rng.random(M) * 0.02 + 1e-3).astype(np.float32)
    ws = (rng.random(N) * 0.02 + 1e-3).astype(np.float32)
    note("int8 gemm M=%d N=%d K=%d %s" % (M, N, K, out_dtype))
    Y = w4.gemm_i8(_t(Xq), _t(xs), _t(Wq), _t(ws), out_dtype)
    torch.cuda.synchronize()
    got = Y.float().cpu().numpy().astype(np.float64)
    ref = oracle_mod.gemm_i8(Xq, xs, Wq, ws)
    bound = REL * np.abs(ref)
    if out_dtype == "bf16":
        bound = bound + np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert np.all(np.abs(got - ref) <= bound + 1e-30)


@pytest.mark.parametrize("ring,K", [(r, 1536) for r in "01234"] + [("3", 1024), ("4", 1024)])
def test_gemm_i8_every_tiling(oracle_mod, monkeypatch, ring, K):
    """Every compiled int8 tiling (0: W4_FORCE_PATH=i8_regs, register-staged;
    W4_I8_RING 1 to 4: the DMA-ring configurations, 3 and 4 splitting K over
    three or two wave groups; at K = 1024 the three-way split falls back) on one ragged case,
    bitwise equal to the default dispatch and within the exact product's
    bound."""
    import torch
    device()
    M, N = 150, 700
    rng = np.random.default_rng(11)
    Xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    Wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    xs = (rng.random(M) * 0.02 + 1e-3).astype(np.float32)
    ws = (rng.random(N) * 0.02 + 1e-3).astype(np.float32)
    note("int8 gemm tiling W4_I8_RING=%s M=%d N=%d K=%d" % (ring, M, N, K))
    Yd = w4.gemm_i8(_t(Xq), _t(xs), _t(Wq), _t(ws), "f32")
    if ring == "0":
        set_dispatch_env(monkeypatch, W4_FORCE_PATH="i8_regs")
    else:
        set_dispatch_env(monkeypatch, W4_I8_RING=ring)
    Y = w4.gemm_i8(_t(Xq), _t(xs), _t(Wq), _t(ws), "f32")
    torch.cuda.synchronize()
    got = Y.cpu().numpy().astype(np.float64)
    ref = oracle_mod.gemm_i8(Xq, xs, Wq, ws)
    assert np.all(np.abs(got - ref) <= REL * np.abs(ref) + 1e-30)
    # the int32 sums are exact and the scales apply in one order: bitwise equal
    assert np.array_equal(Y.cpu().numpy(), Yd.cpu().numpy())


@pytest.mark.parametrize("M", [8, 15, 16, 64, 512])
def test_twin_switch(oracle_mod, M):
    """auto:16 -- below 16 rows the int4 product, at or above the int8 twin:
    equal bit for bit to its two steps, and within the fp32 roundings of the
    oracle's exact W8A8 product of the same quantized operands."""
    import torch
    device()
    N, K, g, blk = 1024, 1536, 256, 512
    W = synth.outlier_weights(N, K, 61)
    Wt = _t(W)
    packed4 = w4.quantize(Wt, g, blk)
    W8, ws8 = w4.quantize_rows_i8(Wt, blk)
    X = synth.draw_activations(np.random.default_rng(M), M, K)
    Xd = to_dev_bf16(X)
    Y = w4.gemm_twin(packed4, W8, ws8, N, K, g, Xd, blk, 16, "f32")
    torch.cuda.synchronize()
    got = Y.cpu().numpy().astype(np.float64)
    if M < 16:
        ref = w4.gemm(packed4, N, K, g, Xd, blk, "f32")
        torch.cuda.synchronize()
        assert np.array_equal(got, ref.cpu().numpy().astype(np.float64))
        return
    Xq, xs = w4.quantize_rows_i8(Xd, blk)
    Y2 = w4.gemm_i8(Xq, xs, W8, ws8, "f32")
    torch.cuda.synchronize()
    assert np.array_equal(got, Y2.cpu().numpy().astype(np.float64))
    Xf = oracle_mod.bf16_to_f64(X).astype(np.float32)
    Xqo, xso = oracle_mod.quantize_rows_i8(Xf, blk)
    Wqo, wso = oracle_mod.quantize_rows_i8(W, blk)
    assert np.array_equal(Xq.cpu().numpy(), Xqo) and np.array_equal(W8.cpu().numpy(), Wqo)
    ref = oracle_mod.gemm_i8(Xqo, xso, Wqo, wso)
    assert np.all(np.abs(got - ref) <= REL * np.abs(ref) + 1e-30)
    # and the twin stays close to the dense product
    dense = Xf.astype(np.float64) @ W.astype(np.float64).T
    assert np.linalg.norm(got - dense) / np.linalg.norm(dense) < 0.02
