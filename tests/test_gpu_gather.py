"""GPU parity of the 4-bit table gather: every output bit against the oracle.

Rows of the embedding-shaped (K = 1536) and per-layer-shaped (K = 8960)
tables, fp32 (exact) and bf16 (round to nearest even), ids with repeats and
out-of-range values (NaN rows), padded output rows, and the full-size tables
of a decode step on sampled ids.
"""
import numpy as np
import pytest

import bit_weight_only_w4a16_amd as w4
from bit_weight_only_w4a16_amd import synth

from _util import device, note, to_dev_bf16, upload_packed

pytestmark = pytest.mark.gpu


def _dev_ids(ids):
    import torch
    return torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(device())


def _bits(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy().view(np.uint32)


def _want_bits(w, dtype):
    return w.view(np.uint16) if dtype == "bf16" else w.view(np.uint32)


def _check(oracle_mod, c, packed, ids, dtype, what):
    import torch
    got = w4.gather(packed, c.N, c.K, c.group, _dev_ids(ids), dtype)
    torch.cuda.synchronize()
    want = oracle_mod.gather(c.P, c.S, c.N, c.K, c.group, ids, dtype)
    g, wb = _bits(got), _want_bits(want, dtype)
    bad = np.argwhere(g != wb)
    assert bad.size == 0, "%s: %d mismatches, first at %s: got %x want %x" % (
        what, len(bad), tuple(bad[0]), g[tuple(bad[0])], wb[tuple(bad[0])])


SHAPES = [(1000, 1536, 32), (700, 8960, 32), (513, 512, 256), (97, 96, 32), (5, 32, 32),
          (300, 1536, 512)]


@pytest.mark.parametrize("N,K,g", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gather_bit_exact(oracle_mod, N, K, g, dtype):
    device()
    c = synth.make_case("table", N, K, g, 1, 600 + N + K, dtype)
    packed = upload_packed(c.P, c.S, N, K, g)
    rng = np.random.default_rng(N + K)
    for B in (1, 7, 33, 257):
        ids = rng.integers(0, N, B).astype(np.int32)
        if B >= 7:
            ids[1] = ids[0]                          # a repeat
            ids[3], ids[5] = -1, N                   # out of range -> NaN rows
            ids[6] = 2 ** 31 - 1
        note("gather N=%d K=%d g=%d B=%d %s" % (N, K, g, B, dtype))
        _check(oracle_mod, c, packed, ids, dtype, "N=%d K=%d B=%d" % (N, K, B))


def test_gather_padded_rows_untouched(oracle_mod):
    import torch
    device()
    N, K, g = 300, 1536, 32
    c = synth.make_case("table", N, K, g, 1, 77, "bf16")
    packed = upload_packed(c.P, c.S, N, K, g)
    ids = np.array([5, 299, 0, 17], dtype=np.int32)
    ldy = K + 64
    Y = torch.full((len(ids), ldy), 3.0, dtype=torch.bfloat16, device=device())
    w4.gather(packed, N, K, g, _dev_ids(ids), "bf16", out=Y[:, :K])
    torch.cuda.synchronize()
    want = oracle_mod.gather(c.P, c.S, N, K, g, ids, "bf16")
    got = _bits(Y)
    assert np.array_equal(got[:, :K], want)
    assert np.all(got[:, K:] == 0x4040)              # 3.0 in bf16, untouched


def test_gather_equals_gemv_columns(oracle_mod):
    """One packed copy serves the lookup and the GEMV: a gathered row n, column
    k equals output n of the GEMV with the one-hot activation e_k (both exact
    in fp32)."""
    import torch
    device()
    N, K, g = 640, 512, 32
    c = synth.make_case("tied", N, K, g, 1, 91, "f32")
    packed = upload_packed(c.P, c.S, N, K, g)
    ids = np.arange(N, dtype=np.int32)
    rows = w4.gather(packed, N, K, g, _dev_ids(ids), "f32")
    for k in (0, 1, 31, 32, 255, 511):
        x = np.zeros(K, dtype=np.uint16)
        x[k] = 0x3F80
        y = w4.gemv(packed, N, K, g, to_dev_bf16(x), "f32")
        torch.cuda.synchronize()
        assert np.array_equal(_bits(y), _bits(rows[:, k].contiguous())), k


@pytest.mark.parametrize("which", ["embed", "ple"])
def test_gather_full_tables_sampled(oracle_mod, which):
    """The decode step's full tables (262144 x 1536 and 262144 x 8960) with
    the 512 ids the benchmark times."""
    device()
    c = synth.lm_head(141) if which == "embed" else synth.ple_table()
    packed = upload_packed(c.P, c.S, c.N, c.K, c.group)
    ids = synth.token_ids(512, 7)
    note("gather full %s table B=512" % which)
    _check(oracle_mod, c, packed, ids, "bf16", which)
    _check(oracle_mod, c, packed, ids[:1], "f32", which + " B=1")
