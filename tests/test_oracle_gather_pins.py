"""Pins of the oracle's bf16 rounding and table gather (CPU only).

The rounding is checked against hand-worked values (nearest neighbour and
both tie directions) and against torch's own float32 -> bfloat16 cast; the
gather against a hand-built table whose rows are written out by hand.
"""
import numpy as np
import pytest

from test_oracle_pins import _pack_from_codes

# (value, bf16 bits), worked by hand: bf16 keeps 8 significant bits.
ROUNDING = [
    (0.0, 0x0000),
    (1.0, 0x3F80),
    (1.0078125, 0x3F81),     # 1 + 2^-7: exact
    (7.0546875, 0x40E2),     # 7 * 1.0078125 = 4 * 1.763671875; 0.763671875 * 128 = 97.75 -> 98
    (3.0234375, 0x4042),     # 3 * 1.0078125: 65.5 units, a tie -> 66 (even)
    (1.01171875, 0x3F82),    # halfway between mantissas 1 (odd) and 2 (even) -> 2
    (1.01953125, 0x3F82),    # halfway between 2 (even) and 3 (odd) -> 2
    (-8.0625, 0xC101),       # -8 * 1.0078125: exact, sign bit set
    (-0.0234375, 0xBCC0),    # -3/128 = -1.5 * 2^-6: exact
    (255.5, 0x4380),         # 255.5 = 1.99609375 * 2^7 -> 255.5 units: tie, 255 odd -> 256
]


@pytest.mark.parametrize("v,bits", ROUNDING)
def test_bf16_rounding_hand_worked(oracle_mod, v, bits):
    assert oracle_mod.f64_to_bf16(v) == bits


def test_bf16_rounding_matches_torch_cast(oracle_mod):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    # values of the gather's form and general normal floats
    codes = rng.integers(-8, 8, 4000).astype(np.float64)
    scales = (rng.integers(0x3A00, 0x4200, 4000).astype(np.uint32) << 16).view(np.float32)
    v = np.concatenate([codes * scales.astype(np.float64),
                        rng.standard_normal(4000).astype(np.float32).astype(np.float64)])
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
    ref = ref.numpy().view(np.uint16)
    got = np.array([oracle_mod.f64_to_bf16(x) for x in v], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_gather_hand_built_table(oracle_mod):
    # N = 3 rows, K = 64 (group 32: two groups per row)
    N, K, g = 3, 64, 32
    C = np.zeros((N, K), dtype=np.int64)
    C[0, :] = 8                      # row 0: all zero
    C[1, :] = np.arange(K) % 16      # row 1: codes 0..15 repeating
    C[2, :32] = 15                   # row 2: +7 then -8
    C[2, 32:] = 0
    S = np.array([[0x3F80, 0x4000],          # 1, 2
                  [0x3F81, 0x3E80],          # 1.0078125, 0.25
                  [0x3F81, 0x3F81]], dtype=np.uint16)
    P = _pack_from_codes(C)
    ids = np.array([1, 2, 0, 5, 1, -1], dtype=np.int32)
    f = oracle_mod.gather(P, S, N, K, g, ids, "f32")
    h = oracle_mod.gather(P, S, N, K, g, ids, "bf16")
    row1 = np.array([(k % 16 - 8) * (1.0078125 if k < 32 else 0.25) for k in range(K)],
                    dtype=np.float32)
    assert np.array_equal(f[0], row1) and np.array_equal(f[4], row1)
    assert np.all(f[1, :32] == np.float32(7 * 1.0078125))
    assert np.all(f[1, 32:] == np.float32(-8 * 1.0078125))
    assert np.all(f[2] == 0.0)
    assert np.all(np.isnan(f[3])) and np.all(np.isnan(f[5]))
    # bf16: row 2 holds 7.0546875 -> 0x40E2 and -8.0625 -> 0xC101
    assert np.all(h[1, :32] == 0x40E2) and np.all(h[1, 32:] == 0xC101)
    assert np.all(h[2] == 0)
    assert np.all(h[3] == 0x7FC0) and np.all(h[5] == 0x7FC0)
    # row 1, code 11 in the first group: 3 * 1.0078125 = 3.0234375 -> tie -> 0x4042
    assert h[0, 11] == 0x4042
    # second group, code 4: -4 * 0.25 = -1 exactly
    assert h[0, 36] == 0xBF80
