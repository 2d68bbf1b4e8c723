"""MI355X (gfx950) W4A16 group-quantized GEMV library: Python binding.

Thin ctypes marshalling over ``libw4a16.so`` (declared in ``include/w4a16.h``):
torch tensors become device pointers plus the current HIP stream.  Every step
of the computation runs in the library's HIP kernels; PyTorch only allocates
device memory and supplies streams.  Importing this package loads nothing; the
library is loaded on first use and a missing or unloadable library raises
``W4LibraryMissing`` (there is no fallback path).

The library follows [P1] "Gemma 4 E2B on a 4 GB GPU with plain PyTorch, faster
than llama.cpp" (the w4gemv.py kernel: packed 4-bit words, groups of 32 with
a bf16 step, value = code - 8, one vector times every weight matrix) and [P2]
"fastgemma -- Gemma 4 E2B, CPU-only, AMX INT8 / AVX-512 VNNI" ("What is in the
file": groups of 256, Hadamard rotation along K with a run-time FWHT).
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a16.so")

W4_OK = 0
W4_F32 = 0
W4_BF16 = 1
W4_SWEEP_GRAPH = 0
W4_SWEEP_PERSISTENT = 1
W4_SWEEP_STREAM = 2

STATUS = {
    0: "W4_OK", -1: "W4_ERR_ARG", -2: "W4_ERR_SHAPE", -3: "W4_ERR_ALIGN",
    -4: "W4_ERR_DTYPE", -5: "W4_ERR_UNSUPPORTED", -6: "W4_ERR_HIP",
    -7: "W4_ERR_NOMEM", -8: "W4_ERR_ARCH", -9: "W4_ERR_TIMEOUT", -10: "W4_ERR_SELFTEST",
}

# every symbol include/w4a16.h declares
EXPORTS = (
    "w4_status_str", "w4_last_error", "w4_device_check", "w4_build_info",
    "w4_packed_bytes", "w4_pack", "w4_pack_host", "w4_unpack_host",
    "w4a16_gemv", "w4a16_gemm_smallM", "w4_fwht", "w4a16_gemm_workspace_bytes",
    "w4a16_gemm", "w4_decode_sweep_create", "w4_decode_sweep_launch",
    "w4_decode_sweep_check", "w4_decode_sweep_info", "w4_decode_sweep_destroy",
    "w4_gather", "w4_quantize", "w4_quantize_rows_i8", "w4_gemm_i8",
    "w4a16_gemm_twin_workspace_bytes", "w4a16_gemm_twin", "w4_attn_workspace_bytes",
    "w4_attn_decode",
    "w4_attn_pack_v", "w4_attn_store_kv", "w4_describe_dispatch", "w4_selftest", "w4_probe_read", "w4_probe_copy", "w4_probe_mfma",
    "w4_probe_handoff", "w4_probe_handoff_bytes",
    "w4a16_gemm_noalloc", "w4a16_gemm_noalloc_max_bytes",
    "w4_config_reload", "w4_tile_table_load",
)


class W4LibraryMissing(RuntimeError):
    pass


class W4Error(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s (%d): %s" % (STATUS.get(status, "?"), status, msg))
        self.status = status


class GemvOp(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("N", ctypes.c_int), ("K", ctypes.c_int),
                ("group", ctypes.c_int), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("y_dtype", ctypes.c_int)]


_lib = None
_lock = threading.Lock()


def lib():
    """The loaded library (raises W4LibraryMissing if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise W4LibraryMissing(
                "libw4a16.so is not built (%s); run "
                "`python -m bit_weight_only_w4a16_amd.build`" % LIB_PATH)
        try:
            L = ctypes.CDLL(LIB_PATH)
        except OSError as e:
            raise W4LibraryMissing("cannot load %s: %s" % (LIB_PATH, e))
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        sig = {
            "w4_status_str": ([i], ctypes.c_char_p),
            "w4_last_error": ([], ctypes.c_char_p),
            "w4_device_check": ([], i),
            "w4_build_info": ([], ctypes.c_char_p),
            "w4_packed_bytes": ([i, i, i], sz),
            "w4_pack": ([vp, vp, i, i, i, vp, vp], i),
            "w4_pack_host": ([vp, vp, i, i, i, vp], i),
            "w4_unpack_host": ([vp, i, i, i, vp, vp], i),
            "w4a16_gemv": ([vp, i, i, i, vp, vp, i, vp], i),
            "w4a16_gemm_smallM": ([vp, i, i, i, i, vp, i, vp, i, i, vp], i),
            "w4_fwht": ([vp, i, vp, i, i, i, i, vp], i),
            "w4a16_gemm_workspace_bytes": ([i, i, i], sz),
            "w4a16_gemm": ([vp, i, i, i, i, vp, i, i, vp, sz, vp, i, i, vp], i),
            "w4_decode_sweep_create": ([ctypes.POINTER(GemvOp), i, i, vp,
                                        ctypes.POINTER(vp)], i),
            "w4_decode_sweep_launch": ([vp, vp], i),
            "w4_decode_sweep_check": ([vp, vp], i),
            "w4_decode_sweep_info": ([vp, ctypes.POINTER(i), ctypes.POINTER(sz),
                                      ctypes.POINTER(i)], i),
            "w4_decode_sweep_destroy": ([vp], i),
            "w4_describe_dispatch": ([i, i, i, i, ctypes.c_char_p, sz], i),
            "w4_config_reload": ([], i),
            "w4_tile_table_load": ([ctypes.c_char_p], i),
            "w4_selftest": ([vp], i),
            "w4_gather": ([vp, i, i, i, vp, i, vp, i, i, vp], i),
            "w4_quantize": ([vp, i, i, i, i, i, i, vp, vp], i),
            "w4_quantize_rows_i8": ([vp, i, i, i, i, i, vp, i, vp, vp], i),
            "w4_gemm_i8": ([vp, i, vp, vp, i, vp, i, i, i, vp, i, i, vp], i),
            "w4a16_gemm_twin_workspace_bytes": ([i, i, i, i], sz),
            "w4a16_gemm_twin": ([vp, vp, i, vp, i, i, i, i, vp, i, i, i, vp, sz, vp, i, i,
                                 vp], i),
            "w4_attn_workspace_bytes": ([i, i], sz),
            "w4_attn_decode": ([vp, vp, i, vp, vp, i, i, i, i, ctypes.c_float, vp, sz, vp, i,
                                vp], i),
            "w4_attn_pack_v": ([vp, i, i, i, vp, vp], i),
            "w4_attn_store_kv": ([vp, vp, i, vp, i, vp, i, vp], i),
            "w4_probe_read": ([vp, sz, vp, vp], i),
            "w4_probe_copy": ([vp, vp, sz, vp], i),
            "w4_probe_mfma": ([i, vp, vp], i),
            "w4_probe_handoff": ([vp, i, i, vp], i),
            "w4_probe_handoff_bytes": ([], sz),
            "w4a16_gemm_noalloc": ([vp, i, i, i, i, vp, i, i, vp, i, i, vp], i),
            "w4a16_gemm_noalloc_max_bytes": ([], sz),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def last_error() -> str:
    return lib().w4_last_error().decode()


def _check(status: int):
    if status != W4_OK:
        raise W4Error(status, last_error())


def _ptr(t) -> ctypes.c_void_p:
    if t is None:
        return ctypes.c_void_p(0)
    if isinstance(t, np.ndarray):
        return ctypes.c_void_p(t.ctypes.data)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None) -> ctypes.c_void_p:
    if stream is not None:
        return ctypes.c_void_p(int(getattr(stream, "cuda_stream", stream)))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(out_dtype: str) -> int:
    if out_dtype in ("f32", "float32"):
        return W4_F32
    if out_dtype in ("bf16", "bfloat16"):
        return W4_BF16
    raise ValueError("out_dtype must be 'f32' or 'bf16'")


def _empty_out(shape, out_dtype, device):
    import torch
    dt = torch.float32 if _dt(out_dtype) == W4_F32 else torch.bfloat16
    return torch.empty(shape, dtype=dt, device=device)


# ------------------------------------------------------------------ info ---

def build_info() -> str:
    return lib().w4_build_info().decode()


def device_check() -> None:
    _check(lib().w4_device_check())


def packed_bytes(N: int, K: int, group: int) -> int:
    return int(lib().w4_packed_bytes(N, K, group))


def describe_dispatch(M: int, N: int, K: int, group: int) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib().w4_describe_dispatch(M, N, K, group, buf, 256))
    return buf.value.decode()


def config_reload() -> None:
    """Re-read W4_TILE_TABLE, W4_FORCE_PATH, W4_LOG and the tuning indices from
    the environment (call after changing them in-process)."""
    _check(lib().w4_config_reload())


def tile_table_load(path=None) -> None:
    """Load a GEMV tile table file (None: remove the loaded table)."""
    _check(lib().w4_tile_table_load(None if path is None else os.fsencode(path)))


def gather(packed, N: int, K: int, group: int, ids, out_dtype: str = "bf16", out=None,
           stream=None):
    """Dequantized rows ids (int32 device tensor [B]) of the packed N x K
    table -> [B, K] fp32 or bf16 tensor (NaN rows for ids outside [0, N))."""
    import torch
    B = int(ids.numel())
    if out is None:
        out = torch.empty((B, K), dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16,
                          device=ids.device)
    _check(lib().w4_gather(_ptr(packed), N, K, group, _ptr(ids), B, _ptr(out), out.stride(0),
                           _dt(out_dtype), _stream(stream)))
    return out


def quantize(W, group: int, had_block: int = 0, out=None, stream=None):
    """Dense fp32 or bf16 weights W [N, K] on the device -> packed uint8 tensor
    (rotated along K by the orthonormal Hadamard blocks of had_block when
    had_block > 0, then int4 with one scale per group)."""
    import torch
    N, K = W.shape
    nb = packed_bytes(N, K, group)
    if out is None:
        out = torch.empty(nb, dtype=torch.uint8, device=W.device)
    wdt = W4_F32 if W.dtype == torch.float32 else (W4_BF16 if W.dtype == torch.bfloat16 else -1)
    _check(lib().w4_quantize(_ptr(W), wdt, W.stride(0), N, K, group, had_block, _ptr(out),
                             _stream(stream)))
    return out


def quantize_rows_i8(X, had_block: int = 0, Q=None, S=None, stream=None):
    """Per-row symmetric int8 of X [N, K] (fp32 or bf16, device) after an
    optional rotation -> (Q int8 [N, K], S fp32 [N])."""
    import torch
    N, K = X.shape
    if Q is None:
        Q = torch.empty((N, K), dtype=torch.int8, device=X.device)
    if S is None:
        S = torch.empty(N, dtype=torch.float32, device=X.device)
    xdt = W4_F32 if X.dtype == torch.float32 else (W4_BF16 if X.dtype == torch.bfloat16 else -1)
    _check(lib().w4_quantize_rows_i8(_ptr(X), xdt, X.stride(0), N, K, had_block, _ptr(Q),
                                     Q.stride(0), _ptr(S), _stream(stream)))
    return Q, S


def gemm_i8(Xq, xs, Wq, ws, out_dtype: str = "bf16", out=None, stream=None):
    """(Xq Wq^T) * xs[m] * ws[n] on the int8 matrix cores."""
    M, K = Xq.shape
    N = Wq.shape[0]
    if out is None:
        out = _empty_out((M, N), out_dtype, Xq.device)
    _check(lib().w4_gemm_i8(_ptr(Xq), Xq.stride(0), _ptr(xs), _ptr(Wq), Wq.stride(0), _ptr(ws),
                            M, N, K, _ptr(out), out.stride(0), _dt(out_dtype), _stream(stream)))
    return out


def gemm_twin(packed4, W8, ws8, N: int, K: int, group: int, X, had_block: int = 0,
              switch_rows: int = 16, out_dtype: str = "bf16", out=None, workspace=None,
              stream=None):
    """The auto:M switch: int4 product below switch_rows rows, the int8 twin
    (activations quantized at run time) at or above."""
    import torch
    M = X.shape[0]
    if out is None:
        out = _empty_out((M, N), out_dtype, X.device)
    ws = int(lib().w4a16_gemm_twin_workspace_bytes(M, K, had_block, switch_rows))
    if workspace is None and ws:
        workspace = torch.empty(ws, dtype=torch.uint8, device=X.device)
    _check(lib().w4a16_gemm_twin(_ptr(packed4), _ptr(W8), W8.stride(0), _ptr(ws8), N, K, group,
                                 M, _ptr(X), X.stride(0), had_block, switch_rows,
                                 _ptr(workspace), ws, _ptr(out), out.stride(0), _dt(out_dtype),
                                 _stream(stream)))
    return out


def attn_workspace_bytes(T: int, D: int) -> int:
    return int(lib().w4_attn_workspace_bytes(T, D))


def attn_pack_v(V, T: int = None, out=None, stream=None):
    """Row-major bf16 V [T, D] (device) -> the blocked layout w4_attn_decode
    reads (a flat bf16 tensor of ceil(T/32)*32*D elements)."""
    import torch
    T = V.shape[0] if T is None else T
    D = V.shape[1]
    if out is None:
        out = torch.empty(((T + 31) // 32) * 32 * D, dtype=torch.bfloat16, device=V.device)
    _check(lib().w4_attn_pack_v(_ptr(V), V.stride(0), T, D, _ptr(out), _stream(stream)))
    return out


def attn_store_kv(k, v, slot: int, K, Vt, stream=None):
    """Writes one slot: K[slot] = k and V slot `slot` = v (blocked layout)."""
    D = K.shape[1]
    _check(lib().w4_attn_store_kv(_ptr(k), _ptr(v), slot, _ptr(K), K.stride(0), _ptr(Vt), D,
                                  _stream(stream)))


def attn_decode(q, K, Vt, T: int, scale: float, pos=None, cur: int = 0, window: int = 0,
                out_dtype: str = "f32", out=None, workspace=None, stream=None):
    """Decode attention of 8 query heads q [8, D] over T slots of one KV head
    (K [>=T, D] row-major, Vt blocked); pos: None or int32 [T] positions."""
    import torch
    D = q.shape[1]
    if out is None:
        out = _empty_out((8, D), out_dtype, q.device)
    ws = attn_workspace_bytes(T, D)
    if workspace is None:
        workspace = torch.empty(ws, dtype=torch.uint8, device=q.device)
    _check(lib().w4_attn_decode(_ptr(q), _ptr(K), K.stride(0), _ptr(Vt), _ptr(pos), T, D, cur,
                                window, float(scale), _ptr(workspace), ws, _ptr(out),
                                _dt(out_dtype), _stream(stream)))
    return out


def selftest(stream=None) -> None:
    """Runs the library's start-up check on the current GPU (raises W4Error)."""
    _check(lib().w4_selftest(_stream(stream)))


# --------------------------------------------------------------- packing ---

def pack(P, S, N: int, K: int, group: int, out=None, stream=None):
    """Canonical codes P (int32/uint32 [N, K/8]) and bf16 scales S (int16 or
    bfloat16 bits [N, K/group]), both on the device -> packed uint8 tensor."""
    import torch
    nb = packed_bytes(N, K, group)
    if out is None:
        out = torch.empty(nb, dtype=torch.uint8, device=P.device)
    _check(lib().w4_pack(_ptr(P), _ptr(S), N, K, group, _ptr(out), _stream(stream)))
    return out


def pack_host(P: np.ndarray, S: np.ndarray, N: int, K: int, group: int) -> np.ndarray:
    P = np.ascontiguousarray(P, dtype=np.uint32)
    S = np.ascontiguousarray(S, dtype=np.uint16)
    nb = packed_bytes(N, K, group)
    if nb == 0:
        raise W4Error(-2, "invalid shape")
    if P.size != N * (K // 8) or S.size != N * (K // group):
        raise ValueError("P or S does not match (N, K, group)")
    out = np.empty(nb, dtype=np.uint8)
    _check(lib().w4_pack_host(_ptr(P), _ptr(S), N, K, group, _ptr(out)))
    return out


def unpack_host(packed: np.ndarray, N: int, K: int, group: int):
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    if packed.size < packed_bytes(N, K, group):
        raise ValueError("packed buffer too small")
    P = np.empty((N, K // 8), dtype=np.uint32)
    S = np.empty((N, K // group), dtype=np.uint16)
    _check(lib().w4_unpack_host(_ptr(packed), N, K, group, _ptr(P), _ptr(S)))
    return P, S


# --------------------------------------------------------------- compute ---

def gemv(packed, N: int, K: int, group: int, x, out_dtype: str = "f32", out=None,
         stream=None):
    """y = W x (M = 1); x: bf16 tensor of K elements on the device."""
    if out is None:
        out = _empty_out((N,), out_dtype, x.device)
    _check(lib().w4a16_gemv(_ptr(packed), N, K, group, _ptr(x), _ptr(out),
                            _dt(out_dtype), _stream(stream)))
    return out


def gemm_smallM(packed, N: int, K: int, group: int, X, out_dtype: str = "bf16",
                out=None, stream=None):
    """Y = X W^T for 2 <= M <= 16 rows; X: bf16 [M, K] (row stride X.stride(0))."""
    M = X.shape[0]
    if out is None:
        out = _empty_out((M, N), out_dtype, X.device)
    _check(lib().w4a16_gemm_smallM(_ptr(packed), N, K, group, M, _ptr(X),
                                   X.stride(0), _ptr(out), out.stride(0),
                                   _dt(out_dtype), _stream(stream)))
    return out


def fwht(X, block: int, out=None, stream=None):
    """Blockwise orthonormal FWHT along K of bf16 X [M, K] -> bf16."""
    import torch
    if out is None:
        out = torch.empty_like(X)
    M, K = X.shape
    _check(lib().w4_fwht(_ptr(X), X.stride(0), _ptr(out), out.stride(0), M, K, block,
                         _stream(stream)))
    return out


def gemm_workspace_bytes(M: int, K: int, had_block: int) -> int:
    return int(lib().w4a16_gemm_workspace_bytes(M, K, had_block))


def gemm(packed, N: int, K: int, group: int, X, had_block: int = 0,
         out_dtype: str = "bf16", out=None, workspace=None, stream=None):
    """Y = FWHT(X) W'^T on the matrix cores (had_block = 0: no transform)."""
    import torch
    M = X.shape[0]
    if out is None:
        out = _empty_out((M, N), out_dtype, X.device)
    ws = gemm_workspace_bytes(M, K, had_block)
    if ws and workspace is None:
        workspace = torch.empty(ws, dtype=torch.uint8, device=X.device)
    _check(lib().w4a16_gemm(_ptr(packed), N, K, group, M, _ptr(X), X.stride(0),
                            had_block, _ptr(workspace), ws, _ptr(out), out.stride(0),
                            _dt(out_dtype), _stream(stream)))
    return out


def gemm_noalloc(packed, N: int, K: int, group: int, X, had_block: int = 0,
                 out_dtype: str = "bf16", out=None, stream=None):
    """w4a16_gemm with the transform output in the library's static device
    array (no workspace, no allocation inside the call)."""
    M = X.shape[0]
    if out is None:
        out = _empty_out((M, N), out_dtype, X.device)
    _check(lib().w4a16_gemm_noalloc(_ptr(packed), N, K, group, M, _ptr(X), X.stride(0),
                                    had_block, _ptr(out), out.stride(0), _dt(out_dtype),
                                    _stream(stream)))
    return out


def gemm_noalloc_max_bytes() -> int:
    return int(lib().w4a16_gemm_noalloc_max_bytes())


class DecodeSweep:
    """A decode step's GEMVs replayed as one graph.  ``ops`` is a list of
    (packed, N, K, group, x, y) with y's dtype (float32 or bfloat16) giving
    the output dtype.  The tensors are borrowed: keep them alive."""

    def __init__(self, ops, mode: int = W4_SWEEP_GRAPH, stream=None):
        import torch
        arr = (GemvOp * len(ops))()
        for j, (packed, N, K, group, x, y) in enumerate(ops):
            dt = W4_F32 if y.dtype == torch.float32 else W4_BF16
            arr[j] = GemvOp(packed.data_ptr(), N, K, group, x.data_ptr(), y.data_ptr(), dt)
        self._keep = list(ops)
        h = ctypes.c_void_p()
        _check(lib().w4_decode_sweep_create(arr, len(ops), mode, _stream(stream),
                                            ctypes.byref(h)))
        self._h = h
        self.mode = mode

    def launch(self, stream=None):
        _check(lib().w4_decode_sweep_launch(self._h, _stream(stream)))

    def check(self, stream=None):
        _check(lib().w4_decode_sweep_check(self._h, _stream(stream)))

    def info(self):
        n, nb, k = ctypes.c_int(), ctypes.c_size_t(), ctypes.c_int()
        _check(lib().w4_decode_sweep_info(self._h, ctypes.byref(n), ctypes.byref(nb),
                                          ctypes.byref(k)))
        return {"n_ops": n.value, "weight_bytes": nb.value, "kernels": k.value}

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            _check(lib().w4_decode_sweep_destroy(self._h))
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------- probes ---

def probe_read(buf, nbytes: int = None, out=None, stream=None):
    """Plain integer sum of a device buffer's 32-bit words (bandwidth probe)."""
    import torch
    if nbytes is None:
        nbytes = buf.numel() * buf.element_size()
    if out is None:
        out = torch.empty(1, dtype=torch.int32, device=buf.device)
    _check(lib().w4_probe_read(_ptr(buf), nbytes, _ptr(out), _stream(stream)))
    return out


def probe_mfma(iters: int, out=None, stream=None):
    """Matrix-core throughput probe: 2048 waves x iters x 16 bf16 MFMAs
    (16384 FLOP each) from registers; returns the (untouched) out buffer."""
    import torch
    if out is None:
        out = torch.zeros(1, dtype=torch.float32, device="cuda")
    _check(lib().w4_probe_mfma(int(iters), _ptr(out), _stream(stream)))
    return out


def probe_handoff(rounds: int, rows: int, work=None, stream=None):
    """Grid-wide handoff probe (``rounds`` rounds, ``rows`` bf16 values per
    workgroup per round); returns the work buffer (uint8), whose first
    32-bit word is nonzero if a poll gave up."""
    import torch
    if work is None:
        work = torch.empty(int(lib().w4_probe_handoff_bytes()), dtype=torch.uint8,
                           device="cuda")
    _check(lib().w4_probe_handoff(_ptr(work), int(rounds), int(rows), _stream(stream)))
    return work


def probe_copy(src, dst, nbytes: int = None, stream=None):
    if nbytes is None:
        nbytes = src.numel() * src.element_size()
    _check(lib().w4_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))
