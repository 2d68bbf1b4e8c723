"""CPU emulation of the kernels' per-chunk arithmetic in fp32, on near-zero
rows (codes all 8 except a few positions, small activations there, large
ones elsewhere), against the fp64 oracle at the acceptance bound.

[P1] "Gemma 4 E2B on a 4 GB GPU with plain PyTorch, faster than llama.cpp",
paragraph on the w4gemv.py kernel: each 4-bit value is made exactly
(value - 8) before it is multiplied.

 - The offset fold sum (128 + c) x - 136 sum x, accumulated in fp32, has a
   rounding error proportional to 136 sum |x|, not to sum |(c - 8) x|: on
   these rows it leaves the bound (the inputs are sharp enough to see it).
 - The fp16 decode ((1024 + c) - 1032, and (1024 + 16 c) / 16 - 72) is exact
   in fp16 arithmetic for every code; the per-slice power-of-two conversion
   of bf16 activations to fp16 round-trips exactly when the slice's nonzero
   magnitudes lie within 2^29 of its largest, and the range test flags the
   slices where it would not.
 - The bf16 decode (nibble at the top of a byte, offset bit flipped, read as
   a signed byte) gives 16 (c - 8) for every code.
 - Exact products accumulated in fp32 (the kernels' order: per chunk two
   chains of pairs, chunks scaled and summed per lane, lanes summed) stay
   within the bound on the same rows.
"""
import numpy as np
import pytest

from bit_weight_only_w4a16_amd import synth

from _util import bound

f32 = np.float32


def _bf16(h):
    return synth.bf16_bits_to_f32(h)


def _case(wide=False):
    return synth.sparse_case("near_zero", 96, 1536, 32, 1, 11, "f32", wide=wide)


def _chunk_sums_fp32(prod):
    """prod [N, C, 32] fp32 exact products -> per-chunk fp32 sums in the
    kernels' order: two chains over the 16 pairs (even pairs, odd pairs),
    each pair added as one dot2 step, then chain 0 + chain 1."""
    N, C, _ = prod.shape
    pairs = prod.reshape(N, C, 16, 2)
    a = [np.zeros((N, C), f32), np.zeros((N, C), f32)]
    for i in range(16):
        j = i & 1
        a[j] = (a[j] + (pairs[:, :, i, 0] + pairs[:, :, i, 1]).astype(f32)).astype(f32)
    return (a[0] + a[1]).astype(f32)


def _lane_sum(chunk_vals, L=16, lane_scale=None):
    """[N, C] fp32 per-chunk contributions -> per-row fp32 totals: lane l
    sums chunks l, l + L, ... in order (then multiplies by its lane_scale),
    then lanes are added pairwise."""
    N, C = chunk_vals.shape
    lanes = np.zeros((N, L), f32)
    for c in range(C):
        lanes[:, c % L] = (lanes[:, c % L] + chunk_vals[:, c]).astype(f32)
    if lane_scale is not None:
        lanes = (lanes * lane_scale[None, :].astype(f32)).astype(f32)
    while lanes.shape[1] > 1:
        h = lanes.shape[1] // 2
        lanes = (lanes[:, :h] + lanes[:, h:]).astype(f32)
    return lanes[:, 0]


def _scales(case):
    return np.repeat(_bf16(case.S), case.group // 32, axis=1).astype(f32)   # [N, C]


def test_fold_arithmetic_fails_on_near_zero_rows(oracle_mod):
    case = _case()
    N, K = case.N, case.K
    codes = oracle_mod.codes(case.P, N, K).astype(np.int64)
    x = _bf16(case.X[0])
    biased = ((128 + codes).astype(f32) * x[None, :]).reshape(N, K // 32, 32)
    off = np.broadcast_to((f32(136) * x).reshape(1, K // 32, 32), biased.shape)
    chunk = (_chunk_sums_fp32(biased) - _chunk_sums_fp32(np.ascontiguousarray(off))).astype(f32)
    y = _lane_sum((_scales(case) * chunk).astype(f32))
    Y, A = oracle_mod.gemm_bf16(case.P, case.S, N, K, 32, case.X)
    err = np.abs(y.astype(np.float64) - Y[0])
    assert (err > bound(Y[0], A[0], "f32")).any(), "the near-zero rows must expose the fold"


def test_fp16_code_decode_is_exact():
    c = np.arange(16)
    h0 = (np.float16(1024) + c.astype(np.float16)).astype(np.float16)   # magic | c
    assert np.array_equal((h0 + np.float16(-1032)).astype(np.float16), (c - 8).astype(np.float16))
    h1 = (np.float16(1024) + (16 * c).astype(np.float16)).astype(np.float16)   # magic | c << 4
    t = (h1 * np.float16(0.0625)).astype(np.float16)
    assert np.array_equal((t + np.float16(-72)).astype(np.float16), (c - 8).astype(np.float16))
    # the bit patterns the and-or forms are those numbers
    assert np.array_equal((0x6400 | c).astype(np.uint16).view(np.float16), h0)
    assert np.array_equal((0x6400 | (c << 4)).astype(np.uint16).view(np.float16), h1)


def test_bf16_code_decode_is_exact():
    c = np.arange(16, dtype=np.uint32)
    byte = ((c << 4) & 0xF0) ^ 0x80
    assert np.array_equal(byte.astype(np.uint8).view(np.int8).astype(np.int64), 16 * (c.astype(np.int64) - 8))


def _to_f16_slice(xs):
    """The kernels' conversion of one lane slice (fp32 copies of bf16 values):
    returns (fp16 values, inverse scale, exact flag)."""
    bits = xs.astype(f32).view(np.uint32) >> 16
    mag = bits & 0x7FFF
    emax = int(mag.max() >> 7)
    nz = mag[mag != 0]
    s = min(142 - emax, 126)
    ok = emax < 255 and (nz.size == 0 or (int(nz.min() >> 7) >= 1 and int(nz.min() >> 7) >= emax - 29))
    h = np.ldexp(xs.astype(np.float64), s).astype(np.float16)
    return h, np.ldexp(1.0, -s), ok


@pytest.mark.parametrize("wide", [False, True])
def test_fp16_activation_conversion(wide):
    case = _case(wide=wide)
    x = _bf16(case.X[0])
    C, L = case.K // 32, 16
    flags = []
    for l in range(L):
        idx = np.concatenate([np.arange(32 * c, 32 * c + 32) for c in range(l, C, L)])
        h, inv, ok = _to_f16_slice(x[idx])
        flags.append(ok)
        if ok:
            assert np.array_equal((h.astype(np.float64) * inv).astype(f32), x[idx])
    assert all(flags) != wide   # the wide case holds a slice the test rejects


def test_exact_products_stay_within_bound(oracle_mod):
    case = _case()
    N, K = case.N, case.K
    codes = oracle_mod.codes(case.P, N, K).astype(np.int64)
    x = _bf16(case.X[0])
    C, L = K // 32, 16
    xh = np.zeros(K, np.float64)
    inv = np.zeros(L)
    for l in range(L):
        idx = np.concatenate([np.arange(32 * c, 32 * c + 32) for c in range(l, C, L)])
        h, iv, ok = _to_f16_slice(x[idx])
        assert ok
        xh[idx] = h.astype(np.float64)
        inv[l] = iv
    prod = ((codes - 8).astype(np.float64) * xh[None, :]).astype(f32)   # exact in fp32
    assert np.array_equal(prod.astype(np.float64), (codes - 8) * xh[None, :])
    chunk = _chunk_sums_fp32(prod.reshape(N, C, 32))
    lane_part = (_scales(case) * chunk).astype(f32)
    y = _lane_sum(lane_part, L, lane_scale=inv)
    Y, A = oracle_mod.gemm_bf16(case.P, case.S, N, K, 32, case.X)
    err = np.abs(y.astype(np.float64) - Y[0])
    b = bound(Y[0], A[0], "f32")
    assert np.all(err <= b), float((err / b).max())
