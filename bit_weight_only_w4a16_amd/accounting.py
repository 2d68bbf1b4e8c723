"""Byte and FLOP accounting for the W4A16 path.

Weight bytes follow the convention the pages' own figures satisfy: each
weight costs its 4-bit code plus its share of the group's 16-bit scale, i.e.
N*K/2 + N*(K/group)*2 bytes, and GB/s uses 1 GB = 1e9 B ([P1] "Gemma 4 E2B on a
4 GB GPU with plain PyTorch, faster than llama.cpp", the summary line of the
w4gemv.py kernel: 1,222.8 MiB per token read in 9.12 ms is 140.6 GB/s).
"""
from __future__ import annotations


def weight_bytes(N: int, K: int, group: int) -> int:
    """Algorithmic weight bytes of an N x K int4 matrix with bf16 group scales."""
    assert K % group == 0
    return N * K // 2 + N * (K // group) * 2


def io_bytes(M: int, N: int, K: int, out_bytes: int) -> int:
    """Activation read plus output write bytes."""
    return M * K * 2 + M * N * out_bytes


def flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def gbps(nbytes: float, seconds: float) -> float:
    return nbytes / seconds / 1e9
