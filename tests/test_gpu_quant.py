"""GPU parity of the rotate-and-quantize packer: every code and scale bit
against the oracle (the same fp32 rotation and rounding rule), on fp32 and
bf16 weights, with and without rotation, ragged and full-size shapes; then
the packed result through the prefill product with the run-time transform
matches the dense product within the quantization bound."""
import numpy as np
import pytest

import bit_weight_only_w4a16_amd as w4
from bit_weight_only_w4a16_amd import synth

from _util import device, note, to_dev_bf16

pytestmark = pytest.mark.gpu

CASES = [  # N, K, group, had_block
    (33, 512, 32, 0), (64, 1536, 256, 512), (100, 1536, 32, 512), (7, 96, 32, 0),
    (5, 768, 256, 256), (65, 2048, 32, 64), (12288, 1536, 256, 512), (1536, 6144, 32, 512),
    (300, 1536, 512, 512), (17, 1024, 512, 0), (40, 640, 32, 128), (9, 1152, 32, 128),
]


def _quantize_both(oracle_mod, W32, N, K, g, blk, wdtype):
    import torch
    if wdtype == "bf16":
        Wt = torch.from_numpy(W32).to(device()).to(torch.bfloat16)
        W32 = Wt.float().cpu().numpy()          # the exact values the GPU sees
    else:
        Wt = torch.from_numpy(W32).to(device())
    packed = w4.quantize(Wt, g, blk)
    torch.cuda.synchronize()
    P, S = w4.unpack_host(packed.cpu().numpy(), N, K, g)
    Po, So = oracle_mod.quantize(W32, g, blk)
    return packed, (P, S), (Po, So)


@pytest.mark.parametrize("N,K,g,blk", CASES)
@pytest.mark.parametrize("wdtype", ["f32", "bf16"])
def test_quantize_bit_exact(oracle_mod, N, K, g, blk, wdtype):
    device()
    note("quantize N=%d K=%d g=%d block=%d %s" % (N, K, g, blk, wdtype))
    W = synth.outlier_weights(N, K, 900 + N + K)
    W[0, :g] = 0.0                               # an all-zero group
    _, (P, S), (Po, So) = _quantize_both(oracle_mod, W, N, K, g, blk, wdtype)
    bad_s = np.argwhere(S != So)
    assert bad_s.size == 0, ("scale", tuple(bad_s[0]), hex(S[tuple(bad_s[0])]),
                             hex(So[tuple(bad_s[0])]))
    bad_p = np.argwhere(P != Po)
    assert bad_p.size == 0, ("codes", tuple(bad_p[0]), hex(P[tuple(bad_p[0])]),
                             hex(Po[tuple(bad_p[0])]))


def test_quantize_padded_rows(oracle_mod):
    import torch
    device()
    N, K, ldw = 40, 1536, 1600
    W = synth.outlier_weights(N, ldw, 31)
    Wt = torch.from_numpy(W).to(device())
    packed = w4.quantize(Wt[:, :K], 256, 512)
    torch.cuda.synchronize()
    P, S = w4.unpack_host(packed.cpu().numpy(), N, K, 256)
    Po, So = oracle_mod.quantize(np.ascontiguousarray(W[:, :K]), 256, 512)
    assert np.array_equal(P, Po) and np.array_equal(S, So)


def test_quantized_prefill_matches_dense(oracle_mod):
    """Offline rotate-and-quantize, then the prefill product with the 512-point
    run-time transform: y ~ W x within the quantization bound, and closer than
    without rotation on weights with outlier channels."""
    import torch
    device()
    N, K, M = 1024, 1536, 64
    W = synth.outlier_weights(N, K, 41)
    X = synth.draw_activations(np.random.default_rng(42), M, K)   # bf16 bits
    Xf = oracle_mod.bf16_to_f64(X)
    Y_dense = Xf @ W.astype(np.float64).T
    Xd = to_dev_bf16(X)
    errs = {}
    for blk in (512, 0):
        packed = w4.quantize(torch.from_numpy(W).to(device()), 256, blk)
        ws = torch.empty(max(1, w4.gemm_workspace_bytes(M, K, blk)), dtype=torch.uint8,
                         device=device())
        Y = w4.gemm(packed, N, K, 256, Xd, blk, "f32", workspace=ws)
        torch.cuda.synchronize()
        Yg = Y.cpu().numpy().astype(np.float64)
        errs[blk] = np.linalg.norm(Yg - Y_dense) / np.linalg.norm(Y_dense)
        if blk:
            P, S = w4.unpack_host(packed.cpu().numpy(), N, K, 256)
            step = np.repeat(oracle_mod.bf16_to_f64(S), 256, axis=1)
            Xr = oracle_mod.fwht(Xf, 512)
            # half a step per weight, the bf16 rounding of the transformed x,
            # and the GEMM's fp32 accumulation
            bound = (np.abs(Xr) @ (0.5 * step).T + 2 ** -8 * np.abs(Xr) @
                     np.abs(oracle_mod.dequant(P, S, N, K, 256)).T + 1e-3)
            assert np.all(np.abs(Yg - Y_dense) <= bound)
    note("prefill rel. error: rotated %.4f, plain %.4f" % (errs[512], errs[0]))
    assert errs[512] < 0.7 * errs[0]
