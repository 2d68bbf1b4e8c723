"""Seeded synthetic inputs for the W4A16 path.

This module only draws random inputs; it holds none of the method's
arithmetic (no decode, no product, no transform), so both the GPU path's tests
and the CPU oracle can take their inputs from it.

Distributions (the same for every workload):
  * packed code words: uniform uint32, i.e. eight i.i.d. uniform 4-bit codes
    0..15 per word, canonical order (element k of a row in word k/8, bits
    [4*(k%8), +4));
  * scales: 0.02*|N(0,1)| + 1e-3 computed in fp32, rounded to bf16 (nearest,
    ties to even), one per (row, K-group);
  * activations: N(0,1) in fp32 rounded to bf16; optionally a fraction of the
    elements (exactly round(frac*M*K), drawn without replacement) multiplied
    by a factor before rounding (outliers).
Draw order per matrix from one ``numpy.random.default_rng(seed)`` (PCG64):
words, then scales, then activations.

Workloads are a stand-in for batch-1 decode of a Gemma-4-E2B-sized model
(hidden 1536, 35 decoder layers, vocabulary 262144), the shapes the pages'
model has; no trained weights are used.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

HIDDEN = 1536
N_LAYERS = 35
VOCAB = 262144

# (name, N, K) of one decoder layer's fused projections, in decode order.
LAYER_SHAPES = (
    ("qkv", 2048 + 256 + 256, HIDDEN),
    ("o", HIDDEN, 2048),
    ("gate_up", 2 * 6144, HIDDEN),
    ("down", HIDDEN, 6144),
)
LM_HEAD_SHAPE = ("lm_head", VOCAB, HIDDEN)
# Per-layer input table: a row of 35 x 256 values per token, 4-bit, group 32.
PLE_WIDTH = N_LAYERS * 256
PLE_SHAPE = ("ple", VOCAB, PLE_WIDTH)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16
    bit patterns.  Inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def draw_weights(rng: np.random.Generator, N: int, K: int, group: int):
    """Canonical packed words P[N][K/8] (uint32) and bf16 scales
    S[N][K/group] (uint16 bit patterns)."""
    assert K % 8 == 0 and K % group == 0
    P = rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint32)
    z = rng.standard_normal(size=(N, K // group), dtype=np.float32)
    s = np.abs(z) * np.float32(0.02) + np.float32(1e-3)
    return P, f32_to_bf16_bits(s)


def draw_activations(rng: np.random.Generator, M: int, K: int,
                     outlier_frac: float = 0.0, outlier_mult: float = 20.0):
    """bf16 activations X[M][K] (uint16 bit patterns)."""
    x = rng.standard_normal(size=(M, K), dtype=np.float32)
    if outlier_frac > 0.0:
        count = int(round(outlier_frac * M * K))
        idx = rng.choice(M * K, size=count, replace=False)
        flat = x.reshape(-1)
        flat[idx] *= np.float32(outlier_mult)
    return f32_to_bf16_bits(x)


@dataclass
class GemvCase:
    name: str
    N: int
    K: int
    group: int
    M: int
    P: np.ndarray        # uint32 [N, K/8] canonical packed codes
    S: np.ndarray        # uint16 [N, K/group] bf16 scales
    X: np.ndarray        # uint16 [M, K] bf16 activations
    out_dtype: str       # "f32" or "bf16"
    seed: int
    hadamard_block: int = 0

    @property
    def weight_bytes(self) -> int:
        """Algorithmic weight bytes: 4-bit codes plus one bf16 scale per group."""
        return self.N * self.K // 2 + self.N * (self.K // self.group) * 2


def make_case(name, N, K, group, M, seed, out_dtype, outlier_frac=0.0,
              hadamard_block=0) -> GemvCase:
    rng = np.random.default_rng(seed)
    P, S = draw_weights(rng, N, K, group)
    X = draw_activations(rng, M, K, outlier_frac=outlier_frac)
    return GemvCase(name, N, K, group, M, P, S, X, out_dtype, seed,
                    hadamard_block)


def codes_to_words(codes: np.ndarray) -> np.ndarray:
    """Canonical packed words of a code matrix [N][K] (values 0..15): element
    k of a row in word k/8, bits [4*(k%8), +4)."""
    N, K = codes.shape
    out = np.zeros((N, K // 8), dtype=np.uint32)
    for j in range(8):
        out |= codes[:, j::8].astype(np.uint32) << np.uint32(4 * j)
    return out


def sparse_case(name, N, K, group, M, seed, out_dtype, small=(1e-3, 1e-2), big=3.0,
                per_chunk=3, wide=False) -> GemvCase:
    """Near-zero rows: every code is 8 (value 0) except at most `per_chunk`
    positions per 32-element chunk (0..per_chunk, uniform per row and chunk;
    every 7th row has exactly one non-8 code in the whole row).  The
    activations are big * N(0,1) everywhere except at four positions per
    chunk, the only places where non-8 codes sit, whose magnitudes are
    uniform in `small` with a random sign.  `wide`: one chunk position per
    row of X instead holds 1e30 and another 1e-10 (a dynamic range far beyond
    fp16's), both at small-activation positions' neighbours."""
    rng = np.random.default_rng(seed)
    C = K // 32
    pos = np.stack([rng.choice(32, size=4, replace=False) for _ in range(C)])   # [C, 4]
    sel = pos + 32 * np.arange(C)[:, None]
    x = (rng.standard_normal(size=(M, K), dtype=np.float32) * np.float32(big))
    mag = rng.uniform(small[0], small[1], size=(M, C, 4)).astype(np.float32)
    sign = np.where(rng.integers(0, 2, size=(M, C, 4)) == 1, 1.0, -1.0).astype(np.float32)
    x[:, sel.reshape(-1)] = (mag * sign).reshape(M, -1)
    if wide:
        for m in range(M):
            c = int(rng.integers(0, C))
            free = [j for j in range(32) if j not in set(pos[c].tolist())]
            a, b = rng.choice(free, size=2, replace=False)
            x[m, 32 * c + a] = np.float32(1e30)
            x[m, 32 * c + b] = np.float32(1e-10)
    # per (row, chunk): 0..per_chunk of the chunk's four small positions
    # (a random subset), each with a code drawn from the 15 non-8 values
    cnt = rng.integers(0, per_chunk + 1, size=(N, C))
    single = (np.arange(N) % 7) == 3
    cnt[single] = 0
    cnt[single, rng.integers(0, C, size=int(single.sum()))] = 1
    perms = np.array(list(__import__("itertools").permutations(range(4))))   # 24 x 4
    rank = perms[rng.integers(0, 24, size=(N, C))]
    take = rank < cnt[:, :, None]
    vals = rng.integers(0, 15, size=(N, C, 4))
    vals = vals + (vals >= 8)
    codes = np.full((N, K), 8, dtype=np.uint8)
    rows = np.broadcast_to(np.arange(N)[:, None, None], take.shape)
    cols = np.broadcast_to(sel[None, :, :], take.shape)
    codes[rows[take], cols[take]] = vals[take]
    P = codes_to_words(codes)
    z = rng.standard_normal(size=(N, K // group), dtype=np.float32)
    S = f32_to_bf16_bits(np.abs(z) * np.float32(0.02) + np.float32(1e-3))
    return GemvCase(name, N, K, group, M, P, S, f32_to_bf16_bits(x), out_dtype, seed)


def layer_seed(layer: int, j: int) -> int:
    return 1 + 4 * layer + j


def single_gemv_small() -> GemvCase:
    """M=1, N=256, K=512, group 32, fp32 out, seed 0."""
    return make_case("gemv_256x512", 256, 512, 32, 1, 0, "f32")


def decoder_layer(layer: int = 0):
    """The four fused projections of one decoder layer, bf16 out."""
    return [make_case(name, N, K, 32, 1, layer_seed(layer, j), "bf16")
            for j, (name, N, K) in enumerate(LAYER_SHAPES)]


def lm_head(seed: int = 0) -> GemvCase:
    """Tied embedding / lm_head GEMV: N=262144, K=1536, group 32, fp32 logits."""
    name, N, K = LM_HEAD_SHAPE
    return make_case(name, N, K, 32, 1, seed, "f32")


def decode_sweep():
    """One decode step's weights: 35 x {qkv, o, gate_up, down} then lm_head,
    a fresh seed per matrix, each with its own activation vector."""
    cases = []
    for layer in range(N_LAYERS):
        cases.extend(decoder_layer(layer))
    cases.append(lm_head(seed=1 + 4 * N_LAYERS))
    return cases


def prefill_g256(M: int) -> GemvCase:
    """Prefill-shaped GEMM: group 256, N=12288, K=1536; activations with 1%
    outliers x20; a 512-point Hadamard rotation along K is applied at run time
    (weights are drawn directly as the stored rotated weights)."""
    return make_case("prefill_g256_M%d" % M, 2 * 6144, HIDDEN, 256, M,
                     1000 + M, "bf16", outlier_frac=0.01, hadamard_block=512)


def ple_table(seed: int = 142) -> GemvCase:
    """Per-layer input table, 262144 x 8960 (35 x 256), group 32 (1.32 GB
    packed).  Its X row is drawn but unused."""
    name, N, K = PLE_SHAPE
    return make_case(name, N, K, 32, 1, seed, "bf16")


def token_ids(B: int, seed: int, vocab: int = VOCAB) -> np.ndarray:
    """B token ids drawn uniformly from [0, vocab) (repeats allowed), int32."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, vocab, B, dtype=np.int64).astype(np.int32)


def outlier_weights(N: int, K: int, seed: int, frac: float = 0.005,
                    factor: float = 20.0) -> np.ndarray:
    """Dense fp32 weights with outlier input channels, the kind a Hadamard
    rotation helps: N(0, 1) entries, then exactly max(1, round(frac * K))
    columns, drawn without replacement, multiplied by `factor`."""
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, K), dtype=np.float32)
    n_out = max(1, int(round(frac * K)))
    cols = rng.choice(K, size=n_out, replace=False)
    W[:, cols] *= np.float32(factor)
    return W
