"""GPU parity of the decode-step sweep: 35 layers x {qkv, o, gate_up, down}
plus the lm_head, every matrix with its own seed and activation, replayed as
one graph.  Every one of the 141 outputs is checked against the oracle, and a
second replay must give identical bits."""
import numpy as np
import pytest

import bit_weight_only_w4a16_amd as w4
from bit_weight_only_w4a16_amd import synth

from _util import (assert_within, device, from_dev, note, set_dispatch_env, to_dev_bf16,
                   upload_packed)

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


# "persistent_inline": the decode-ordered kernel with every resident share
# decoded while multiplying (W4_FORCE_PATH ordered_inline) instead of ahead
MODES = [("graph", w4.W4_SWEEP_GRAPH), ("persistent", w4.W4_SWEEP_PERSISTENT),
         ("persistent_inline", w4.W4_SWEEP_PERSISTENT), ("stream", w4.W4_SWEEP_STREAM)]


@pytest.fixture(autouse=True)
def _mode_env(request, monkeypatch):
    """Selects the inline decode for the persistent_inline cases."""
    cs = getattr(request.node, "callspec", None)
    name = cs.params.get("name", "") if cs else ""
    if name.endswith("_inline"):
        set_dispatch_env(monkeypatch, W4_FORCE_PATH="ordered_inline")


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


def _column(oracle_mod, c, k):
    """Column k of a group-32 case's dequantized weights, from the oracle's
    dequantization of the 32-element chunk that holds k."""
    q = k // 32
    Pq = np.ascontiguousarray(c.P[:, 4 * q:4 * q + 4])
    Sq = np.ascontiguousarray(c.S[:, q:q + 1])
    return oracle_mod.dequant(Pq, Sq, c.N, 32, 32)[:, k % 32].astype(np.float32)


@pytest.mark.parametrize("name,mode", MODES)
def test_sweep_one_hot_is_bit_exact(oracle_mod, sweep_data, name, mode):
    """Every one of the 141 ops with a one-hot activation and fp32 output:
    each output is exactly (code - 8) * scale of the hot column, through
    the stream kernel (the headline), the decode-ordered kernel and the
    graph of GEMV kernels."""
    import torch
    cases, ops = sweep_data
    rng = np.random.default_rng(17)
    ks, probe = [], []
    for j, (c, op) in enumerate(zip(cases, ops)):
        k = [0, c.K - 1, int(rng.integers(0, c.K))][j % 3]
        x = torch.zeros(c.K, dtype=torch.bfloat16, device=device())
        x[k] = 1.0
        y = torch.full((c.N,), float("nan"), dtype=torch.float32, device=device())
        probe.append((op[0], c.N, c.K, c.group, x, y))
        ks.append(k)
    note("one-hot sweep mode=%s" % name)
    sw = w4.DecodeSweep(probe, mode)
    sw.launch()
    sw.check()
    torch.cuda.synchronize()
    for c, k, op in zip(cases, ks, probe):
        got = from_dev(op[5])
        assert np.array_equal(got.view(np.uint32), _column(oracle_mod, c, k).view(np.uint32)), \
            (name, c.name, c.seed, k)
    sw.close()


@pytest.mark.parametrize("name,mode", MODES[:3])
def test_chained_ops_read_the_previous_output(oracle_mod, name, mode):
    """Decode order: op i + 1 multiplies op i's bf16 output (square 1536 x
    1536 weights, x_{i+1} = y_i), outputs NaN-filled before every replay, so
    an op that read its input before the previous op finished writing it
    would see NaN.  Each y_i is checked against the oracle applied to the
    GPU's own y_{i-1}."""
    import torch
    device()
    n_ops, N = 12, 1536
    cases, ys = [], []
    x0b = synth.draw_activations(np.random.default_rng(4), 1, N)[0]
    x0 = to_dev_bf16(x0b)
    ops = []
    for i in range(n_ops):
        c = synth.make_case("chain%d" % i, N, N, 32, 1, 300 + i, "bf16")
        y = torch.full((N,), float("nan"), dtype=torch.bfloat16, device=device())
        ops.append((upload_packed(c.P, c.S, N, N, 32), N, N, 32, x0 if i == 0 else ys[-1], y))
        cases.append(c)
        ys.append(y)
    note("chained sweep mode=%s ops=%d" % (name, n_ops))
    sw = w4.DecodeSweep(ops, mode)
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        sw.launch()
        sw.check()
        torch.cuda.synchronize()
        xin = x0b
        for i, c in enumerate(cases):
            got = ys[i].view(torch.int16).cpu().numpy().view(np.uint16)
            Y, A = oracle_mod.gemm_bf16(c.P, c.S, N, N, 32, xin, threads=16)
            assert_within(synth.bf16_bits_to_f32(got), Y, A, "bf16",
                          "%s rep %d op %d" % (name, rep, i))
            xin = got
    sw.close()


def test_decoded_ahead_equals_inline(sweep_data, monkeypatch, capfd):
    """The decode-ordered kernel's two ways of decoding a resident share
    (ahead into registers, or while multiplying) run the same tasks in the
    same order: all 141 outputs are bitwise equal.  W4_LOG names which way
    each handle runs."""
    import torch
    cases, ops = sweep_data
    got = {}
    for name, force in (("ahead", ""), ("inline", "ordered_inline")):
        set_dispatch_env(monkeypatch, W4_FORCE_PATH=force, W4_LOG="1")
        note("persistent sweep, resident shares decoded %s" % name)
        for op in ops:
            op[5].fill_(float("nan"))
        sw = w4.DecodeSweep(ops, w4.W4_SWEEP_PERSISTENT)
        sw.launch()
        sw.check()
        torch.cuda.synchronize()
        got[name] = [from_dev(op[5]).copy() for op in ops]
        sw.close()
        err = capfd.readouterr().err
        assert ("resident shares decoded %s" % name) in err, err
    for c, a, b in zip(cases, got["ahead"], got["inline"]):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), c.name


@pytest.mark.parametrize("force", ["", "ordered_inline"])
def test_persistent_gives_up_and_recovers(oracle_mod, monkeypatch, force):
    """The decode-ordered kernel's give-up path: with no completion polls
    allowed (W4_SWEEP_POLL_LIMIT=0) every workgroup stops at its second op,
    the kernel ends normally, and the check reports W4_ERR_TIMEOUT and resets
    the counters; a handle created with the default limit then replays the
    same ops correctly."""
    import torch
    device()
    n_ops, N = 4, 1536
    x0b = synth.draw_activations(np.random.default_rng(9), 1, N)[0]
    x0 = to_dev_bf16(x0b)
    cases, ys, ops = [], [], []
    for i in range(n_ops):
        c = synth.make_case("giveup%d" % i, N, N, 32, 1, 900 + i, "bf16")
        y = torch.full((N,), float("nan"), dtype=torch.bfloat16, device=device())
        ops.append((upload_packed(c.P, c.S, N, N, 32), N, N, 32, x0 if i == 0 else ys[-1], y))
        cases.append(c)
        ys.append(y)
    set_dispatch_env(monkeypatch, W4_SWEEP_POLL_LIMIT="0", W4_FORCE_PATH=force)
    note("persistent sweep give-up force=%r" % force)
    sw = w4.DecodeSweep(ops, w4.W4_SWEEP_PERSISTENT)
    sw.launch()
    with pytest.raises(w4.W4Error) as err:
        sw.check()
    assert err.value.status == -9
    sw.close()
    monkeypatch.delenv("W4_SWEEP_POLL_LIMIT")
    w4.config_reload()
    sw = w4.DecodeSweep(ops, w4.W4_SWEEP_PERSISTENT)
    for y in ys:
        y.fill_(float("nan"))
    torch.cuda.synchronize()
    sw.launch()
    sw.check()
    torch.cuda.synchronize()
    xin = x0b
    for i, c in enumerate(cases):
        got = ys[i].view(torch.int16).cpu().numpy().view(np.uint16)
        Y, A = oracle_mod.gemm_bf16(c.P, c.S, N, N, 32, xin, threads=16)
        assert_within(synth.bf16_bits_to_f32(got), Y, A, "bf16", "after give-up op %d" % i)
        xin = got
    sw.close()
