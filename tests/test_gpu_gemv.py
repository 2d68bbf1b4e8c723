"""GPU parity of the batch-1 GEMV (w4a16_gemv) and the packer against the
fp64 oracle: the small 256 x 512 case, one decoder layer's four fused
projections, the 262144 x 1536 lm_head, ragged and edge shapes, the one-hot
dequantization probe (bit-exact), determinism and output guard regions."""
import numpy as np
import pytest

import bit_weight_only_w4a16_amd as w4
from bit_weight_only_w4a16_amd import synth

from _util import (assert_within, device, from_dev, note, set_dispatch_env, to_dev_bf16,
                   to_dev_u16, to_dev_u32, upload_packed)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    device()
    w4.device_check()


def _run_case(oracle_mod, case, out_dtype=None, threads=8):
    out_dtype = out_dtype or case.out_dtype
    note("gemv %s N=%d K=%d g=%d out=%s" % (case.name, case.N, case.K, case.group, out_dtype))
    packed = upload_packed(case.P, case.S, case.N, case.K, case.group)
    x = to_dev_bf16(case.X[0])
    y = w4.gemv(packed, case.N, case.K, case.group, x, out_dtype)
    Y, A = oracle_mod.gemm_bf16(case.P, case.S, case.N, case.K, case.group, case.X[0],
                                threads=threads)
    return assert_within(from_dev(y), Y, A, out_dtype, case.name), packed, x, y


def test_device_pack_equals_host_pack():
    for (N, K, g) in [(256, 512, 32), (33, 96, 32), (97, 1536, 256), (1, 32, 32)]:
        rng = np.random.default_rng(N + K)
        P, S = synth.draw_weights(rng, N, K, g)
        dev = upload_packed(P, S, N, K, g).cpu().numpy()
        host = w4.pack_host(P, S, N, K, g)
        nc = N * K // 2
        off = w4.packed_bytes(N, K, g) - ((N * (K // g) * 2 + 255) // 256 * 256)
        assert np.array_equal(dev[:nc], host[:nc])
        assert np.array_equal(dev[off:off + N * (K // g) * 2], host[off:off + N * (K // g) * 2])


def test_small_case_f32_and_bf16(oracle_mod):
    case = synth.single_gemv_small()
    r, _, _, _ = _run_case(oracle_mod, case, "f32")
    note("  worst err/bound = %.3g" % r)
    _run_case(oracle_mod, case, "bf16")


def test_one_hot_dequant_is_bit_exact(oracle_mod):
    """x = e_k gives y[n] = (code(n,k) - 8) * scale(n, k/32) exactly, for every
    k of the 256 x 512 case, through the production kernel."""
    import torch
    case = synth.single_gemv_small()
    N, K = case.N, case.K
    packed = upload_packed(case.P, case.S, N, K, 32)
    W = oracle_mod.dequant(case.P, case.S, N, K, 32).astype(np.float32)
    X = torch.zeros((K, K), dtype=torch.bfloat16, device=device())
    X.fill_diagonal_(1.0)
    Y = torch.empty((K, N), dtype=torch.float32, device=device())
    for k in range(K):
        w4.gemv(packed, N, K, 32, X[k], "f32", out=Y[k])
    got = Y.cpu().numpy()
    assert np.array_equal(got.T, W)


@pytest.mark.parametrize("layer", [0, 34])
def test_decoder_layer_shapes(oracle_mod, layer):
    for case in synth.decoder_layer(layer):
        r, _, _, _ = _run_case(oracle_mod, case)
        note("  worst err/bound = %.3g" % r)


def test_one_hot_sampled_on_layer_shapes(oracle_mod):
    import torch
    for case in synth.decoder_layer(0)[1:2] + synth.decoder_layer(0)[3:4]:
        N, K = case.N, case.K
        packed = upload_packed(case.P, case.S, N, K, 32)
        rng = np.random.default_rng(5)
        ks = sorted(set([0, K - 1] + rng.integers(0, K, 14).tolist()))
        for k in ks:
            x = torch.zeros(K, dtype=torch.bfloat16, device=device())
            x[k] = 1.0
            y = from_dev(w4.gemv(packed, N, K, 32, x, "f32"))
            col = np.array([oracle_mod.weight(case.P, case.S, K, 32, n, k)
                            for n in range(0, N, 97)], dtype=np.float32)
            assert np.array_equal(y[::97], col), (case.name, k)


def test_lm_head_full(oracle_mod):
    case = synth.lm_head()
    r, _, _, _ = _run_case(oracle_mod, case, threads=16)
    note("  worst err/bound = %.3g" % r)


RAGGED = [(1, 32, 32), (3, 64, 32), (33, 96, 32), (65, 288, 32), (97, 1056, 32),
          (1000, 2048, 32), (7, 6144, 32), (129, 16384, 32), (5, 20000, 32),
          (31, 256, 256), (65, 1536, 256), (17, 512, 256), (4097, 1536, 32),
          (2, 160, 32), (63, 4096, 256),
          # group 512 (the int4 g512 build): odd and even group counts per row
          (100, 1536, 512), (33, 1024, 512), (12288, 1536, 512), (65, 6144, 512),
          # the largest K the calls accept (2^20)
          (3, 1 << 20, 32), (2, 1 << 20, 512),
          # large N on the contiguous-range kernel, ragged row groups and ranges
          (262141, 1536, 32), (65539, 6144, 32)]


@pytest.mark.parametrize("N,K,g", RAGGED)
def test_ragged_shapes(oracle_mod, N, K, g):
    case = synth.make_case("ragged", N, K, g, 1, N * 7 + K, "f32")
    _run_case(oracle_mod, case)
    _run_case(oracle_mod, case, "bf16")


def test_degenerate_values(oracle_mod):
    """All-8 codes give exact zeros; a zero activation gives zeros; large
    activations stay in tolerance."""
    import torch
    N, K = 77, 1536
    P = np.full((N, K // 8), 0x88888888, dtype=np.uint32)
    rng = np.random.default_rng(1)
    _, S = synth.draw_weights(rng, N, K, 32)
    packed = upload_packed(P, S, N, K, 32)
    x = to_dev_bf16(synth.draw_activations(rng, 1, K)[0])
    assert np.all(from_dev(w4.gemv(packed, N, K, 32, x, "f32")) == 0.0)
    P2, S2 = synth.draw_weights(rng, N, K, 32)
    packed2 = upload_packed(P2, S2, N, K, 32)
    z = torch.zeros(K, dtype=torch.bfloat16, device=device())
    assert np.all(from_dev(w4.gemv(packed2, N, K, 32, z, "f32")) == 0.0)
    xb = synth.draw_activations(rng, 1, K, outlier_frac=0.05, outlier_mult=1000.0)[0]
    y = from_dev(w4.gemv(packed2, N, K, 32, to_dev_bf16(xb), "f32"))
    Y, A = oracle_mod.gemm_bf16(P2, S2, N, K, 32, xb)
    assert_within(y, Y, A, "f32", "large activations")


def test_deterministic_bitwise():
    case = synth.decoder_layer(0)[2]
    packed = upload_packed(case.P, case.S, case.N, case.K, 32)
    x = to_dev_bf16(case.X[0])
    a = from_dev(w4.gemv(packed, case.N, case.K, 32, x, "f32"))
    for _ in range(3):
        b = from_dev(w4.gemv(packed, case.N, case.K, 32, x, "f32"))
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_output_guard_regions(oracle_mod):
    import torch
    for out_dtype, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        for (N, K) in [(33, 96), (2560, 1536)]:
            case = synth.make_case("guard", N, K, 32, 1, 3, out_dtype)
            packed = upload_packed(case.P, case.S, N, K, 32)
            G = 64
            buf = torch.empty(N + 2 * G, dtype=tdt, device=device())
            buf.fill_(-12345.0)
            before = from_dev(buf)
            w4.gemv(packed, N, K, 32, to_dev_bf16(case.X[0]), out_dtype, out=buf[G:G + N])
            h = from_dev(buf)
            assert np.array_equal(h[:G], before[:G]) and np.array_equal(h[G + N:], before[G + N:])
            Y, A = oracle_mod.gemm_bf16(case.P, case.S, N, K, 32, case.X[0])
            assert_within(h[G:G + N], Y, A, out_dtype, "guard")


def test_selftest_passes():
    """The library's own start-up check (closed-form one-hot outputs)."""
    device()
    w4.selftest()


def test_probes_run():
    """The bandwidth and matrix-core probes run and report what they state:
    the read probe's integer sum, the copy, and an MFMA probe that writes
    nothing."""
    import torch
    device()
    buf = torch.arange(1 << 16, dtype=torch.int32, device=device())
    s = w4.probe_read(buf)
    torch.cuda.synchronize()
    expect = int(np.arange(1 << 16, dtype=np.int64).sum() % (1 << 32))
    assert (int(s.item()) & 0xFFFFFFFF) == expect
    dst = torch.empty_like(buf)
    w4.probe_copy(buf, dst)
    out = torch.full((1,), 7.0, dtype=torch.float32, device=device())
    w4.probe_mfma(4, out)
    torch.cuda.synchronize()
    assert torch.equal(dst, buf)
    assert out.item() == 7.0


def test_output_on_input_is_refused():
    """An output that shares bytes with the activation or the weights is
    refused with W4_ERR_ARG before anything is launched, and the buffers are
    left as they were."""
    import torch
    case = synth.single_gemv_small()
    packed = w4.pack(torch.from_numpy(case.P.view(np.int32)).to(device()),
                     torch.from_numpy(case.S.view(np.int16)).to(device()),
                     case.N, case.K, case.group)
    buf = torch.zeros(case.K + case.N, dtype=torch.bfloat16, device=device())
    buf[:case.K] = torch.from_numpy(case.X[0].view(np.int16)).to(device()).view(torch.bfloat16)
    before = buf.clone()
    with pytest.raises(w4.W4Error) as e:
        w4.gemv(packed, case.N, case.K, case.group, buf[:case.K], "bf16", out=buf[8:8 + case.N])
    assert e.value.status == -1
    with pytest.raises(w4.W4Error) as e:
        w4.gemv(packed, case.N, case.K, case.group, buf[:case.K], "bf16",
                out=packed.view(torch.bfloat16)[:case.N])
    assert e.value.status == -1
    torch.cuda.synchronize()
    assert torch.equal(buf, before)
    # adjacent, not overlapping: runs
    y = w4.gemv(packed, case.N, case.K, case.group, buf[:case.K], "bf16", out=buf[case.K:])
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all()


@pytest.mark.parametrize("rows", [0, 1, 6, 24, 64])
def test_handoff_probe(rows):
    """The handoff probe completes every round (no poll gave up) and leaves
    in each of its two vectors what its last round on that vector wrote:
    r + j at element w * rows + j (r the round, w the workgroup)."""
    import torch
    device()
    rounds = 7
    work = w4.probe_handoff(rounds, rows)
    torch.cuda.synchronize()
    h = work.cpu().numpy()
    assert int(h[:4].view(np.uint32)[0]) == 0
    if rows == 0:
        return
    n = 256 * rows
    vec = 256 * 64 * 2
    for buf, last in ((0, rounds - 1 if (rounds - 1) % 2 == 0 else rounds - 2),
                      (1, rounds - 1 if (rounds - 1) % 2 == 1 else rounds - 2)):
        y = h[2048 + buf * vec: 2048 + buf * vec + 2 * n].view(np.uint16)
        expect = (last + np.tile(np.arange(rows), 256)).astype(np.uint16)
        assert np.array_equal(y, expect), buf


@pytest.mark.parametrize("path", ["", "gemv_contig"])
def test_one_hot_through_the_lm_head(oracle_mod, monkeypatch, path):
    """x = e_k through the 262144 x 1536 lm_head (its searched tile, and the
    contiguous-range kernel): every output is exactly (code - 8) * scale of
    column k."""
    import torch
    set_dispatch_env(monkeypatch, W4_FORCE_PATH=path)
    case = synth.lm_head()
    N, K = case.N, case.K
    assert ("contiguous" in w4.describe_dispatch(1, N, K, 32)) == bool(path)
    packed = upload_packed(case.P, case.S, N, K, 32)
    for k in (0, 1, 31, 32, 777, K - 1):
        x = torch.zeros(K, dtype=torch.bfloat16, device=device())
        x[k] = 1.0
        y = from_dev(w4.gemv(packed, N, K, 32, x, "f32"))
        q = k // 32
        col = oracle_mod.dequant(np.ascontiguousarray(case.P[:, 4 * q:4 * q + 4]),
                                 np.ascontiguousarray(case.S[:, q:q + 1]), N, 32, 32)[:, k % 32]
        assert np.array_equal(y.view(np.uint32), col.astype(np.float32).view(np.uint32)), k


# One table entry per tile feature the heuristic never picks: three stages
# (strided and contiguous rows), one and two waves per workgroup, explicit
# grids (one workgroup; more waves than row groups), 8 lanes per row, the
# generic loop at 16 lanes, and the contiguous kernel on a ragged row count.
TABLE_CASES = [
    ("gemv 2560 1536 32 16 3 4 77 3 0", "bf16"),
    ("gemv 1536 2048 32 32 2 1 0 3 0", "bf16"),
    ("gemv 1000 6144 32 64 3 2 1 2 0", "f32"),
    ("gemv 333 1536 32 8 6 4 4096 2 0", "f32"),
    ("gemv 4097 2048 32 16 4 2 300 3 0", "bf16"),
    ("gemv 777 1024 256 16 0 4 9 2 0", "f32"),
    ("gemv 70001 1536 32 16 3 4 0 3 1", "f32"),
    ("gemv 70001 1024 32 32 1 4 97 3 1", "bf16"),
]


@pytest.mark.parametrize("line,odt", TABLE_CASES)
def test_table_tiles_parity(oracle_mod, tmp_path, line, odt):
    """Every tile feature a table can ask for, through w4a16_gemv, against the
    oracle; outputs past N untouched."""
    import torch
    f = tmp_path / "tiles.txt"
    f.write_text(line + "\n")
    N, K, g = (int(v) for v in line.split()[1:4])
    w4.tile_table_load(str(f))
    try:
        assert "(table)" in w4.describe_dispatch(1, N, K, g)
        note("table tile %s out=%s" % (line, odt))
        case = synth.make_case("table", N, K, g, 1, N + K, odt)
        packed = upload_packed(case.P, case.S, N, K, g)
        x = to_dev_bf16(case.X[0])
        dt = torch.float32 if odt == "f32" else torch.bfloat16
        ybuf = torch.full((N + 64,), float("nan"), dtype=dt, device=device())
        w4.gemv(packed, N, K, g, x, odt, out=ybuf[:N])
        torch.cuda.synchronize()
        Y, A = oracle_mod.gemm_bf16(case.P, case.S, N, K, g, case.X[0], threads=16)
        assert_within(from_dev(ybuf[:N]), Y, A, odt, line)
        assert np.isnan(from_dev(ybuf[N:])).all()
    finally:
        w4.tile_table_load(None)
