"""Oracle for the W4A16 path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, scalar fp64 CPU implementation (``oracle.c``) of what the GPU
library computes, written from the pages' definitions and sharing no code with
the GPU path.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package; the product path never does.

Functions follow:
  * [P1] "Gemma 4 E2B on a 4 GB GPU with plain PyTorch, faster than llama.cpp",
    the paragraph introducing the compressed-tensors W4A16 checkpoint (groups
    of 32, bf16 step per group) and the paragraph on the w4gemv.py kernel
    (packed 4-bit words, value = code - 8, exact);
  * [P2] "fastgemma -- Gemma 4 E2B, CPU-only, AMX INT8 / AVX-512 VNNI",
    section "What is in the file" (W' = W H^T with a runtime fast
    Walsh-Hadamard transform of the activation; int4 groups of 256).

Every function here is pinned by a CPU test to something other than itself
(hand-typed tables, closed forms, brute force with library matmul, invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_OUT_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_OUT_DIR, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (-O2, no explicit SIMD, OpenMP over rows)."""
    os.makedirs(_OUT_DIR, exist_ok=True)
    stale = (not os.path.exists(_LIB_PATH)
             or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC))
    if force or stale:
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c99",
               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            i = ctypes.c_int
            lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
            lib.oracle_bf16_to_f64.restype = ctypes.c_double
            lib.oracle_bf16_array_to_f64.argtypes = [P, P, ctypes.c_size_t]
            lib.oracle_code.argtypes = [P, i, i, i]
            lib.oracle_code.restype = i
            lib.oracle_codes.argtypes = [P, i, i, P]
            lib.oracle_weight.argtypes = [P, P, i, i, i, i]
            lib.oracle_weight.restype = ctypes.c_double
            lib.oracle_dequant.argtypes = [P, P, i, i, i, P]
            lib.oracle_gemm.argtypes = [P, P, i, i, i, P, i, i, P, P, i]
            lib.oracle_fwht.argtypes = [P, P, i, i, i]
            lib.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
            lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
            lib.oracle_gather.argtypes = [P, P, i, i, i, P, i, i, P]
            lib.oracle_quantize.argtypes = [P, i, i, i, i, i, P, P]
            lib.oracle_quantize_rows_i8.argtypes = [P, i, i, i, i, P, P]
            lib.oracle_gemm_i8.argtypes = [P, P, P, P, i, i, i, P]
            lib.oracle_attn_decode.argtypes = [P, P, P, P, i, i, i, i, i, ctypes.c_double,
                                               P, P]
            _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def bf16_to_f64(h) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    h = _c(h, np.uint16)
    out = np.empty(h.shape, dtype=np.float64)
    _load().oracle_bf16_array_to_f64(_ptr(h), _ptr(out), h.size)
    return out


def code(P, K: int, n: int, k: int) -> int:
    P = _c(P, np.uint32)
    return int(_load().oracle_code(_ptr(P), K, n, k))


def codes(P, N: int, K: int) -> np.ndarray:
    """All 4-bit codes (0..15) of the canonical packed matrix, N x K int8."""
    P = _c(P, np.uint32)
    assert P.size == N * (K // 8)
    out = np.empty((N, K), dtype=np.int8)
    _load().oracle_codes(_ptr(P), N, K, _ptr(out))
    return out


def weight(P, S, K: int, group: int, n: int, k: int) -> float:
    P = _c(P, np.uint32)
    S = _c(S, np.uint16)
    return float(_load().oracle_weight(_ptr(P), _ptr(S), K, group, n, k))


def dequant(P, S, N: int, K: int, group: int) -> np.ndarray:
    """Dense fp64 W[n][k] = (code - 8) * scale (exact)."""
    P = _c(P, np.uint32)
    S = _c(S, np.uint16)
    assert P.size == N * (K // 8) and S.size == N * (K // group)
    W = np.empty((N, K), dtype=np.float64)
    _load().oracle_dequant(_ptr(P), _ptr(S), N, K, group, _ptr(W))
    return W


def gemm(P, S, N: int, K: int, group: int, X, threads: int = 1):
    """Y[m][n] = sum_k w(n,k) X[m][k] in fp64, sequential k; also
    A[m][n] = sum_k |w(n,k) X[m][k]|.  X is float64 (M x K) or (K,)."""
    P = _c(P, np.uint32)
    S = _c(S, np.uint16)
    X = _c(X, np.float64)
    squeeze = X.ndim == 1
    X2 = X.reshape(1, K) if squeeze else X
    M = X2.shape[0]
    assert X2.shape[1] == K
    assert P.size == N * (K // 8) and S.size == N * (K // group)
    Y = np.empty((M, N), dtype=np.float64)
    A = np.empty((M, N), dtype=np.float64)
    _load().oracle_gemm(_ptr(P), _ptr(S), N, K, group, _ptr(X2), M, K,
                        _ptr(Y), _ptr(A), int(threads))
    if squeeze:
        return Y[0], A[0]
    return Y, A


def gemm_bf16(P, S, N: int, K: int, group: int, Xbf16, threads: int = 1):
    """gemm() with bf16 activations (uint16 bit patterns), widened exactly."""
    return gemm(P, S, N, K, group, bf16_to_f64(Xbf16), threads)


def fwht(X, block: int) -> np.ndarray:
    """Blockwise orthonormal Sylvester-order FWHT along the last axis (fp64)."""
    X = _c(X, np.float64)
    squeeze = X.ndim == 1
    X2 = X.reshape(1, -1) if squeeze else X
    M, K = X2.shape
    assert block > 0 and block & (block - 1) == 0 and K % block == 0
    out = np.empty_like(X2)
    _load().oracle_fwht(_ptr(X2), _ptr(out), M, K, block)
    return out[0] if squeeze else out


def f64_to_bf16(v: float) -> int:
    """bf16 bit pattern of v, round to nearest even (v zero or bf16-normal)."""
    return int(_load().oracle_f64_to_bf16(float(v)))


def gather(P, S, N: int, K: int, group: int, ids, out_dtype: str = "f32") -> np.ndarray:
    """Rows ids of the dequantized N x K table: float32 [B, K] (exact) or
    uint16 bf16 bit patterns [B, K] (round to nearest even); NaN rows for
    ids outside [0, N)."""
    P = _c(P, np.uint32)
    S = _c(S, np.uint16)
    ids = _c(ids, np.int32)
    B = ids.shape[0]
    bf = out_dtype == "bf16"
    out = np.empty((B, K), dtype=np.uint16 if bf else np.float32)
    _load().oracle_gather(_ptr(P), _ptr(S), N, K, group, _ptr(ids), B, 1 if bf else 0,
                          _ptr(out))
    return out


def quantize(W, group: int, block: int = 0):
    """Rotate (block > 0: orthonormal FWHT per block along K, fp32) and
    quantize the fp32 matrix W [N, K] -> (canonical codes P [N, K/8] uint32,
    bf16 scales S [N, K/group] uint16)."""
    W = _c(W, np.float32)
    N, K = W.shape
    assert K % group == 0 and (block == 0 or K % block == 0)
    P = np.empty((N, K // 8), dtype=np.uint32)
    S = np.empty((N, K // group), dtype=np.uint16)
    _load().oracle_quantize(_ptr(W), N, K, K, group, block, _ptr(P), _ptr(S))
    return P, S


def attn_decode(q, K, V, scale: float, pos=None, cur: int = 0, window: int = 0):
    """Decode attention over T cache slots: q [H, D], K and V [T, D] as bf16
    bit patterns (uint16); pos: None (every slot valid) or int32 [T] slot
    positions (valid: 0 <= pos <= cur and, window > 0, pos > cur - window).
    Returns (out [H, D], absout [H, D]) in fp64."""
    q = _c(q, np.uint16)
    K = _c(K, np.uint16)
    V = _c(V, np.uint16)
    H, D = q.shape
    T = K.shape[0]
    assert K.shape == (T, D) and V.shape == (T, D)
    pp = None if pos is None else _c(pos, np.int32)
    out = np.empty((H, D))
    absout = np.empty((H, D))
    _load().oracle_attn_decode(_ptr(q), _ptr(K), _ptr(V),
                               None if pp is None else _ptr(pp), H, T, D, cur, window,
                               float(scale), _ptr(out), _ptr(absout))
    return out, absout


def quantize_rows_i8(W, block: int = 0):
    """Per-row symmetric int8 of the fp32 matrix W [N, K] after an optional
    fp32 rotation (block > 0) -> (Q int8 [N, K], S fp32 [N])."""
    W = _c(W, np.float32)
    N, K = W.shape
    assert block == 0 or K % block == 0
    Q = np.empty((N, K), dtype=np.int8)
    S = np.empty(N, dtype=np.float32)
    _load().oracle_quantize_rows_i8(_ptr(W), N, K, K, block, _ptr(Q), _ptr(S))
    return Q, S


def gemm_i8(Xq, xs, Wq, ws) -> np.ndarray:
    """(Xq Wq^T) * xs[m] * ws[n]: exact integer sums, fp64 scaling."""
    Xq = _c(Xq, np.int8)
    Wq = _c(Wq, np.int8)
    xs = _c(xs, np.float32)
    ws = _c(ws, np.float32)
    M, K = Xq.shape
    N = Wq.shape[0]
    Y = np.empty((M, N))
    _load().oracle_gemm_i8(_ptr(Xq), _ptr(xs), _ptr(Wq), _ptr(ws), M, N, K, _ptr(Y))
    return Y
