"""GPU parity of the decode-step sweep: 35 layers x {qkv, o, gate_up, down}
plus the lm_head, every matrix with its own seed and activation, replayed as
one graph.  Every one of the 141 outputs is checked against the oracle, and a
second replay must give identical bits."""
import numpy as np
import pytest

import bit_weight_only_w4a16_amd as w4
from bit_weight_only_w4a16_amd import synth

from _util import assert_within, device, from_dev, note, to_dev_bf16, upload_packed

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sweep_data(oracle_mod):
    import torch
    device()
    w4.device_check()
    cases = synth.decode_sweep()
    ops, refs = [], []
    for c in cases:
        packed = upload_packed(c.P, c.S, c.N, c.K, c.group)
        x = to_dev_bf16(c.X[0])
        dt = torch.float32 if c.out_dtype == "f32" else torch.bfloat16
        y = torch.full((c.N,), float("nan"), dtype=dt, device=device())
        ops.append((packed, c.N, c.K, c.group, x, y))
    torch.cuda.synchronize()
    return cases, ops


def _check_all(oracle_mod, cases, ops, what):
    worst = 0.0
    for c, op in zip(cases, ops):
        Y, A = oracle_mod.gemm_bf16(c.P, c.S, c.N, c.K, c.group, c.X[0], threads=16)
        worst = max(worst, assert_within(from_dev(op[5]), Y, A, c.out_dtype,
                                         "%s %s seed %d" % (what, c.name, c.seed)))
    return worst


MODES = [("graph", w4.W4_SWEEP_GRAPH), ("persistent", w4.W4_SWEEP_PERSISTENT),
         ("stream", w4.W4_SWEEP_STREAM)]


@pytest.mark.parametrize("name,mode", MODES)
def test_sweep_all_outputs(oracle_mod, sweep_data, name, mode):
    import torch
    cases, ops = sweep_data
    note("sweep mode=%s ops=%d" % (name, len(ops)))
    for op in ops:
        op[5].fill_(float("nan"))
    try:
        sw = w4.DecodeSweep(ops, mode)
    except w4.W4Error as e:
        if e.status == -5:
            pytest.skip("mode not built: %s" % e)
        raise
    info = sw.info()
    assert info["n_ops"] == 141
    assert info["weight_bytes"] == 923_222_016
    sw.launch()
    sw.check()
    torch.cuda.synchronize()
    worst = _check_all(oracle_mod, cases, ops, name)
    note("  worst err/bound = %.3g" % worst)
    first = [from_dev(op[5]).copy() for op in ops]
    # every replay recomputes every output: NaN-fill between replays
    for rep in range(3):
        for op in ops:
            op[5].fill_(float("nan"))
        torch.cuda.synchronize()
        sw.launch()
        sw.check()
        torch.cuda.synchronize()
        for a, op in zip(first, ops):
            b = from_dev(op[5])
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (rep, op[1], op[2])
    sw.close()


# Ragged shapes: row counts that end inside a 64-row output block, blocks
# shared by several waves (more waves than tiles), every compiled tile shape
# of the one-kernel modes, and K with an odd number of groups per row (the
# generic loop).  Outputs past each op's N must stay untouched.
RAGGED_OPS = [(33, 512, 32, "f32"), (100, 1536, 32, "bf16"), (1000, 2048, 32, "bf16"),
              (4097, 1536, 32, "f32"), (65, 6144, 32, "bf16"), (130, 96, 32, "f32"),
              (77, 768, 256, "bf16"), (5000, 1536, 32, "bf16"), (1, 1536, 32, "f32"),
              (129, 3072, 32, "bf16"), (63, 1024, 32, "f32"), (31, 64, 32, "bf16"),
              (50, 4096, 32, "f32"), (70, 1536, 512, "bf16"), (40, 1024, 512, "f32")]


@pytest.mark.parametrize("name,mode", MODES)
def test_sweep_ragged_shapes(oracle_mod, name, mode):
    import torch
    device()
    w4.device_check()
    cases, ops, guards = [], [], []
    for j, (N, K, g, odt) in enumerate(RAGGED_OPS):
        c = synth.make_case("ragged%d" % j, N, K, g, 1, 500 + j, odt)
        dt = torch.float32 if odt == "f32" else torch.bfloat16
        # one extra element after the outputs, which nothing may write
        ybuf = torch.full((N + 1,), float("nan"), dtype=dt, device=device())
        guards.append(ybuf)
        ops.append((upload_packed(c.P, c.S, N, K, g), N, K, g, to_dev_bf16(c.X[0]), ybuf[:N]))
        cases.append(c)
    note("ragged sweep mode=%s ops=%d" % (name, len(ops)))
    try:
        sw = w4.DecodeSweep(ops, mode)
    except w4.W4Error as e:
        if e.status == -5:
            pytest.skip("mode not built: %s" % e)
        raise
    for rep in range(2):
        for op in ops:
            op[5].fill_(float("nan"))
        torch.cuda.synchronize()
        sw.launch()
        sw.check()
        torch.cuda.synchronize()
        _check_all(oracle_mod, cases, ops, "%s rep %d" % (name, rep))
        for gbuf in guards:
            assert np.isnan(from_dev(gbuf[-1:]))[0], "write past N"
    sw.close()


@pytest.mark.parametrize("bpc", ["1", "3"])
def test_sweep_stream_other_grids(oracle_mod, monkeypatch, bpc):
    """The stream partition at other workgroup counts per CU (equal shares
    instead of the four-round weighting): every output still computed once
    and correct, on the ragged op list."""
    import torch
    device()
    monkeypatch.setenv("W4_SWEEP_BLOCKS_PER_CU", bpc)
    cases, ops = [], []
    for j, (N, K, g, odt) in enumerate(RAGGED_OPS):
        c = synth.make_case("grid%d" % j, N, K, g, 1, 700 + j, odt)
        dt = torch.float32 if odt == "f32" else torch.bfloat16
        y = torch.full((N,), float("nan"), dtype=dt, device=device())
        ops.append((upload_packed(c.P, c.S, N, K, g), N, K, g, to_dev_bf16(c.X[0]), y))
        cases.append(c)
    note("stream sweep blocks per CU %s ops=%d" % (bpc, len(ops)))
    sw = w4.DecodeSweep(ops, w4.W4_SWEEP_STREAM)
    sw.launch()
    sw.check()
    torch.cuda.synchronize()
    _check_all(oracle_mod, cases, ops, "stream bpc %s" % bpc)
    sw.close()
