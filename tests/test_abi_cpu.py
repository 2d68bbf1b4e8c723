"""C-ABI checks that need no GPU: the library loads, exports every symbol its
header declares, rejects bad arguments before any HIP call, and the host
packer is the documented bijection."""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_weight_only_w4a16_amd as w4
from bit_weight_only_w4a16_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(w4.LIB_PATH):
        from bit_weight_only_w4a16_amd import build
        build.build(verbose=False)
    return w4.lib()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(w4[a-z0-9_A-Z]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_symbol(L):
    names = _declared_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), n
    assert sorted(w4.EXPORTS) == names


def test_status_strings(L):
    for code, name in w4.STATUS.items():
        s = L.w4_status_str(code).decode()
        assert s and s != "unknown status", (code, name)
    assert L.w4_status_str(-1000).decode() == "unknown status"


def test_packed_bytes(L):
    assert w4.packed_bytes(256, 512, 32) == 65536 + 8192
    # codes then scales, each padded to 256 bytes
    assert w4.packed_bytes(1, 32, 32) == 256 + 256
    assert w4.packed_bytes(262144, 1536, 32) == 201326592 + 25165824
    assert w4.packed_bytes(12288, 1536, 256) == 9437184 + 147456
    for bad in [(0, 512, 32), (16, 48, 32), (16, 512, 64), (16, 256, 512), (-1, 32, 32)]:
        assert w4.packed_bytes(*bad) == 0


VP = ctypes.c_void_p
A16 = VP(0x10000)   # aligned, never dereferenced: validation fails first
A2 = VP(0x10002)


@pytest.mark.parametrize("args,status", [
    ((A16, 256, 512, 64, A16, A16, 0), -2),       # group
    ((A16, 256, 1024, 1024, A16, A16, 0), -2),    # group 1024
    ((A16, 256, 768, 512, A16, A16, 0), -2),      # K % 512
    ((A16, 0, 512, 32, A16, A16, 0), -2),         # N
    ((A16, 256, 500, 32, A16, A16, 0), -2),       # K % group
    ((A16, 256, 512, 32, A16, A16, 7), -4),       # dtype
    ((VP(0), 256, 512, 32, A16, A16, 0), -1),     # null packed
    ((A16, 256, 512, 32, VP(0), A16, 0), -1),     # null x
    ((A16, 256, 512, 32, A16, VP(0), 0), -1),     # null y
    ((A2, 256, 512, 32, A16, A16, 0), -3),        # misaligned packed
    ((A16, 256, 512, 32, A2, A16, 0), -3),        # misaligned x
    ((A16, 256, 512, 32, A16, A2, 0), -3),        # fp32 y misaligned
])
def test_gemv_validation(L, args, status):
    st = L.w4a16_gemv(*args, VP(0))
    assert st == status, w4.last_error()
    assert w4.last_error()


def test_smallm_validation(L):
    f = L.w4a16_gemm_smallM
    assert f(A16, 64, 512, 32, 1, A16, 512, A16, 64, 1, VP(0)) == -2   # M < 2
    assert f(A16, 64, 512, 32, 17, A16, 512, A16, 64, 1, VP(0)) == -2  # M > 16
    assert f(A16, 64, 512, 32, 4, A16, 500, A16, 64, 1, VP(0)) == -2   # ldx < K
    assert f(A16, 64, 512, 32, 4, A16, 516, A16, 64, 1, VP(0)) == -3   # ldx % 8
    assert f(A16, 64, 512, 32, 4, A16, 512, A16, 60, 1, VP(0)) == -2   # ldy < N


def test_gather_validation(L):
    f = L.w4_gather
    assert f(A16, 64, 512, 48, A16, 4, A16, 512, 1, VP(0)) == -2     # group
    assert f(A2, 64, 512, 32, A16, 4, A16, 512, 1, VP(0)) == -3      # packed alignment
    assert f(A16, 64, 512, 32, A16, -1, A16, 512, 1, VP(0)) == -2    # B < 0
    assert f(A16, 64, 512, 32, VP(0), 4, A16, 512, 1, VP(0)) == -1   # ids NULL
    assert f(A16, 64, 512, 32, A2, 4, A16, 512, 1, VP(0)) == -3      # ids alignment
    assert f(A16, 64, 512, 32, A16, 4, A2, 512, 1, VP(0)) == -3      # Y alignment
    assert f(A16, 64, 512, 32, A16, 4, A16, 500, 1, VP(0)) == -2     # ldy < K
    assert f(A16, 64, 512, 32, A16, 4, A16, 516, 1, VP(0)) == -3     # bf16 rows misaligned
    assert f(A16, 64, 512, 32, A16, 4, A16, 514, 0, VP(0)) == -3     # fp32 rows misaligned
    assert f(A16, 64, 512, 32, A16, 4, A16, 512, 7, VP(0)) == -4     # dtype
    # B = 0 launches nothing
    assert f(A16, 64, 512, 32, VP(0), 0, VP(0), 512, 1, VP(0)) == 0


def test_quantize_validation(L):
    f = L.w4_quantize
    assert f(A16, 0, 512, 64, 512, 48, 0, A16, VP(0)) == -2      # group
    assert f(A16, 2, 512, 64, 512, 32, 0, A16, VP(0)) == -4      # W dtype
    assert f(A16, 0, 512, 64, 512, 32, 384, A16, VP(0)) == -2    # had_block
    assert f(A16, 0, 1536, 64, 1536, 32, 1024, A16, VP(0)) == -2  # had_block > 512
    assert f(A16, 0, 768, 64, 768, 32, 512, A16, VP(0)) == -2    # K % had_block
    assert f(A2, 0, 512, 64, 512, 32, 0, A16, VP(0)) == -3       # W alignment
    assert f(A16, 0, 512, 64, 512, 32, 0, A2, VP(0)) == -3       # packed alignment
    assert f(A16, 0, 500, 64, 512, 32, 0, A16, VP(0)) == -2      # ldw < K
    assert f(A16, 0, 514, 64, 512, 32, 0, A16, VP(0)) == -3      # fp32 rows misaligned
    assert f(A16, 1, 516, 64, 512, 32, 0, A16, VP(0)) == -3      # bf16 rows misaligned
    assert f(VP(0), 0, 512, 64, 512, 32, 0, A16, VP(0)) == -1    # W NULL


def test_attention_validation(L):
    f = L.w4_attn_decode
    F = ctypes.c_float
    ws = L.w4_attn_workspace_bytes(1000, 512)
    assert ws == 32 * (32 + 8 * 512) * 4                   # ceil(1000/32) = 32 slices
    assert L.w4_attn_workspace_bytes(1000, 384) == 0
    assert L.w4_attn_workspace_bytes(1 << 20, 256) == 256 * (32 + 8 * 256) * 4   # at most 256 slices
    ok = (A16, A16, 512, A16, VP(0), 1000, 512, 999, 0, F(0.04), A16, ws, A16, 0, VP(0))

    def call(**kw):
        args = list(ok)
        names = ["q", "K", "ldk", "Vt", "pos", "T", "D", "cur", "window", "scale", "ws",
                 "ws_bytes", "out", "odt", "s"]
        for k, v in kw.items():
            args[names.index(k)] = v
        return f(*args)

    assert call(D=384) == -2
    assert call(T=0) == -2
    assert call(q=A2) == -3
    assert call(Vt=A2) == -3
    assert call(ldk=500) == -3
    assert call(ldk=516) == -3
    assert call(pos=A2) == -3
    assert call(window=-1) == -1
    assert call(scale=F(float("nan"))) == -1
    assert call(ws_bytes=ws - 1) == -2
    assert call(odt=5) == -4
    assert L.w4_attn_pack_v(A16, 500, 100, 512, A16, VP(0)) == -2     # ldv < D
    assert L.w4_attn_pack_v(A16, 512, 100, 512, A2, VP(0)) == -3
    assert L.w4_attn_store_kv(A16, A16, -1, A16, 512, A16, 512, VP(0)) == -2
    assert L.w4_attn_store_kv(A16, A16, 3, A16, 100, A16, 512, VP(0)) == -2


def test_int8_validation(L):
    q = L.w4_quantize_rows_i8
    assert q(A16, 2, 512, 4, 512, 0, A16, 512, A16, VP(0)) == -4      # dtype
    assert q(A16, 0, 512, 4, 100, 0, A16, 512, A16, VP(0)) == -2      # K % 8
    assert q(A16, 0, 512, 4, 512, 384, A16, 512, A16, VP(0)) == -2    # had_block
    assert q(A16, 0, 512, 4, 512, 0, A16, 516, A16, VP(0)) == -3      # ldq % 8
    assert q(A16, 0, 512, 4, 512, 0, A16, 512, VP(0), VP(0)) == -1    # S NULL
    assert q(A2, 0, 512, 4, 512, 0, A16, 512, A16, VP(0)) == -3       # X alignment
    g = L.w4_gemm_i8
    assert g(A16, 512, A16, A16, 512, A16, 4, 64, 500, A16, 64, 1, VP(0)) == -2   # K % 128
    assert g(A16, 520, A16, A16, 512, A16, 4, 64, 512, A16, 64, 1, VP(0)) == -3   # ldx % 16
    assert g(A16, 512, VP(0), A16, 512, A16, 4, 64, 512, A16, 64, 1, VP(0)) == -1  # xs NULL
    assert g(A16, 512, A16, A16, 512, A16, 4, 64, 512, A16, 60, 1, VP(0)) == -2   # ldy < N
    assert g(A16, 512, A16, A16, 512, A16, 0, 64, 512, A16, 64, 1, VP(0)) == -2   # M = 0
    t = L.w4a16_gemm_twin
    assert L.w4a16_gemm_twin_workspace_bytes(64, 1536, 512, 16) == 64 * 1536 + 64 * 4
    assert L.w4a16_gemm_twin_workspace_bytes(8, 1536, 512, 16) == 8 * 1536 * 2
    assert t(A16, A16, 1536, A16, 64, 1536, 256, 64, A16, 1536, 512, 0, A16, 1 << 20, A16, 64,
             1, VP(0)) == -1                                            # switch_rows
    assert t(A16, A16, 1536, A16, 64, 1536, 256, 64, A16, 1536, 512, 16, A16, 100, A16, 64,
             1, VP(0)) == -2                                            # workspace
    assert t(A16, VP(0), 1536, A16, 64, 1536, 256, 64, A16, 1536, 512, 16, A16, 1 << 20, A16,
             64, 1, VP(0)) == -1                                        # twin NULL


def test_fwht_validation(L):
    f = L.w4_fwht
    assert f(A16, 1536, A16, 1536, 4, 1536, 384, VP(0)) == -2    # not a power of 2
    assert f(A16, 1536, A16, 1536, 4, 1536, 2048, VP(0)) == -2   # too large
    assert f(A16, 1536, A16, 1536, 4, 1000, 512, VP(0)) == -2    # K % block
    assert f(A16, 1536, A16, 1544, 4, 1536, 512, VP(0)) == -1    # in place, strides differ
    assert f(A2, 1536, A16, 1536, 4, 1536, 512, VP(0)) == -3


def test_gemm_validation(L):
    f = L.w4a16_gemm
    assert f(A16, 64, 1536, 256, 64, A16, 1536, 384, A16, 1 << 20, A16, 64, 1, VP(0)) == -2
    assert f(A16, 64, 1536, 256, 64, A16, 1536, 512, A16, 100, A16, 64, 1, VP(0)) == -2
    assert f(A16, 64, 1536, 256, 0, A16, 1536, 0, VP(0), 0, A16, 64, 1, VP(0)) == -2
    assert f(A16, 64, 1536, 256, 64, A16, 1536, 512, A2, 1 << 20, A16, 64, 1, VP(0)) == -3
    assert w4.gemm_workspace_bytes(512, 1536, 512) == 512 * 1536 * 2
    assert w4.gemm_workspace_bytes(512, 1536, 0) == 0


def test_gemm_noalloc_validation(L):
    """Bad arguments and a transform larger than the static array are
    rejected before any HIP call (this machine has no GPU)."""
    f = L.w4a16_gemm_noalloc
    assert L.w4a16_gemm_noalloc_max_bytes() == 8 << 20
    assert f(VP(0), 64, 1536, 256, 64, A16, 1536, 512, A16, 64, 1, VP(0)) == -1    # NULL
    assert f(A16, 64, 1536, 256, 64, A16, 1536, 384, A16, 64, 1, VP(0)) == -2      # had_block
    assert f(A16, 64, 1536, 256, 64, A2, 1536, 512, A16, 64, 1, VP(0)) == -3       # X align
    M = (8 << 20) // (1536 * 2) + 1
    assert f(A16, 64, 1536, 256, M, A16, 1536, 512, A16, 64, 1, VP(0)) == -2       # too big
    assert "static scratch" in w4.last_error()


def test_sweep_validation(L):
    ops = (w4.GemvOp * 2)()
    ops[0] = w4.GemvOp(0x10000, 64, 512, 32, 0x10000, 0x10000, 0)
    ops[1] = w4.GemvOp(0x10000, 64, 512, 48, 0x10000, 0x10000, 0)
    h = ctypes.c_void_p()
    assert L.w4_decode_sweep_create(ops, 2, 0, VP(0), ctypes.byref(h)) == -2
    assert "op 1" in w4.last_error()
    ops[1] = w4.GemvOp(0x10002, 64, 512, 32, 0x10000, 0x10000, 0)
    assert L.w4_decode_sweep_create(ops, 2, 0, VP(0), ctypes.byref(h)) == -3
    assert L.w4_decode_sweep_create(ops, 2, 9, VP(0), ctypes.byref(h)) == -1
    assert L.w4_decode_sweep_create(ops, 0, 0, VP(0), ctypes.byref(h)) == -1
    assert L.w4_decode_sweep_launch(VP(0), VP(0)) == -1
    assert L.w4_decode_sweep_destroy(VP(0)) == -1


def test_outputs_must_not_overlap_inputs(L):
    """An output that shares a byte with the activations or the weights of
    its product is refused before any HIP call (other workgroups still read
    them while outputs are written)."""
    if L.w4_device_check() != -6:
        pytest.skip("a HIP device is present: the fake-pointer calls would launch")
    P, X, Y = VP(0x100000), VP(0x200000), VP(0x300000)   # disjoint fake buffers
    nb = L.w4_packed_bytes(256, 512, 32)
    assert L.w4a16_gemv(P, 256, 512, 32, X, Y, 0, VP(0)) == -6          # validates, no device
    assert L.w4a16_gemv(P, 256, 512, 32, X, X, 0, VP(0)) == -1          # y on x
    assert L.w4a16_gemv(P, 256, 512, 32, X, VP(0x200000 + 1022), 1, VP(0)) == -1  # last byte
    assert L.w4a16_gemv(P, 256, 512, 32, X, VP(0x200000 + 1024), 1, VP(0)) == -6  # adjacent
    assert L.w4a16_gemv(P, 256, 512, 32, X, VP(0x100000 + nb - 4), 0, VP(0)) == -1  # on weights
    assert L.w4a16_gemm_smallM(P, 256, 512, 32, 4, X, 512, VP(0x200000 + 3 * 1024), 256, 1,
                               VP(0)) == -1                              # Y on X's last row
    assert L.w4a16_gemm(P, 256, 512, 32, 64, X, 512, 0, VP(0), 0, VP(0x200000 + 64 * 1024 - 2),
                        256, 1, VP(0)) == -1                             # Y on X's last element
    assert L.w4a16_gemm_noalloc(P, 256, 512, 32, 64, X, 512, 0, X, 256, 1, VP(0)) == -1
    ops = (w4.GemvOp * 2)()
    ops[0] = w4.GemvOp(0x100000, 256, 512, 32, 0x200000, 0x300000, 0)
    ops[1] = w4.GemvOp(0x400000, 256, 512, 32, 0x300000, 0x200000, 1)   # x = y of op 0: allowed
    h = ctypes.c_void_p()
    ops[1] = w4.GemvOp(0x400000, 256, 512, 32, 0x300000, 0x300000, 1)   # y on its own x
    assert L.w4_decode_sweep_create(ops, 2, 1, VP(0), ctypes.byref(h)) == -1
    assert "op 1" in w4.last_error()
    ops[1] = w4.GemvOp(0x400000, 256, 512, 32, 0x300000, 0x100000 + 64, 1)  # on op 0's weights
    assert L.w4_decode_sweep_create(ops, 2, 1, VP(0), ctypes.byref(h)) == -1
    assert "weights of op 0" in w4.last_error()


def test_probe_validation(L):
    assert L.w4_probe_read(A16, 0, A16, VP(0)) == -2
    assert L.w4_probe_read(A16, 24, A16, VP(0)) == -2
    assert L.w4_probe_read(A2, 32, A16, VP(0)) == -3
    assert L.w4_probe_copy(A16, A2, 32, VP(0)) == -3
    assert L.w4_probe_mfma(0, A16, VP(0)) == -2
    assert L.w4_probe_mfma((1 << 20) + 1, A16, VP(0)) == -2
    assert L.w4_probe_mfma(8, VP(0), VP(0)) == -1
    assert L.w4_probe_mfma(8, A2, VP(0)) == -3
    assert L.w4_probe_handoff_bytes() >= 2048 + 2 * 256 * 64 * 2
    assert L.w4_probe_handoff(VP(0), 1, 6, VP(0)) == -1
    assert L.w4_probe_handoff(VP(0x10010), 1, 6, VP(0)) == -3
    assert L.w4_probe_handoff(VP(0x10000), 0, 6, VP(0)) == -2
    assert L.w4_probe_handoff(VP(0x10000), (1 << 20) + 1, 6, VP(0)) == -2
    assert L.w4_probe_handoff(VP(0x10000), 1, -1, VP(0)) == -2
    assert L.w4_probe_handoff(VP(0x10000), 1, 65, VP(0)) == -2


def test_describe_dispatch_tile_table(L, monkeypatch):
    # the model's shapes: the built-in (searched) table
    for shape in [(12288, 1536, 32), (262144, 1536, 32), (1536, 6144, 32), (2560, 1536, 32),
                  (1536, 2048, 32), (256, 512, 32)]:
        assert w4.describe_dispatch(1, *shape).endswith("(built-in table)"), shape
    # the heuristic for the same shapes: zero-waste lane splits
    from _util import set_dispatch_env
    set_dispatch_env(monkeypatch, W4_FORCE_PATH="gemv_tiled")
    assert w4.describe_dispatch(1, 12288, 1536, 32).startswith("gemv L=16 U=3")
    assert w4.describe_dispatch(1, 262144, 1536, 32).startswith("gemv L=16 U=3")
    assert w4.describe_dispatch(1, 1536, 6144, 32).startswith("gemv L=64 U=3")
    assert w4.describe_dispatch(1, 2560, 1536, 32).startswith("gemv L=16 U=3")
    assert w4.describe_dispatch(1, 256, 512, 32).startswith("gemv L=16 U=1")
    set_dispatch_env(monkeypatch, W4_FORCE_PATH="")
    # K = 128: 4 chunks, 8 lanes per row with half of them masked
    assert w4.describe_dispatch(1, 100, 128, 32).startswith("gemv L=8 U=1")
    # an odd number of groups per row (3) takes the generic loop: the tiled
    # loop reads scales as dword pairs
    assert w4.describe_dispatch(1, 100, 96, 32).startswith("gemv_generic")
    assert w4.describe_dispatch(1, 100, 768, 256).startswith("gemv_generic")
    assert w4.describe_dispatch(1, 100, 20000, 32).startswith("gemv_generic")
    # 2..32 rows (8..32 at group 32) of a matrix of >= 128 48-row tiles with
    # K a multiple of 512 up to 2048: the split-K kernel, one or two
    # activation tiles
    assert w4.describe_dispatch(2, 12288, 1536, 256).startswith("splitk mfma 16x16x32 rows 48 x 1 ")
    assert w4.describe_dispatch(16, 12288, 1536, 256).startswith("splitk mfma 16x16x32 rows 48 x 1 ")
    assert w4.describe_dispatch(17, 12288, 1536, 256).startswith("splitk mfma 16x16x32 rows 48 x 2 ")
    assert w4.describe_dispatch(32, 12288, 1536, 512).startswith("splitk mfma 16x16x32 rows 48 x 2 ")
    assert w4.describe_dispatch(8, 12288, 1536, 32).startswith("splitk")
    assert w4.describe_dispatch(32, 12288, 1536, 32).startswith("splitk")
    assert "(512 each)" in w4.describe_dispatch(8, 6144, 2048, 256)
    # fewer than 128 tiles, or K past 2048: the small-M kernels
    assert w4.describe_dispatch(8, 2560, 1536, 256).startswith("smallm")
    assert w4.describe_dispatch(9, 2560, 1536, 256).startswith("smallm mfma")
    assert w4.describe_dispatch(16, 2560, 1536, 256).startswith("smallm mfma")
    assert w4.describe_dispatch(8, 2560, 1536, 32).startswith("smallm mfma")
    assert w4.describe_dispatch(8, 12288, 3072, 256).startswith("smallm mfma")
    # W4_FORCE_PATH=no_splitk: the kernels those shapes take otherwise
    set_dispatch_env(monkeypatch, W4_FORCE_PATH="no_splitk")
    assert w4.describe_dispatch(9, 12288, 1536, 256).startswith("smallm mfma")
    assert w4.describe_dispatch(16, 12288, 1536, 32).startswith("smallm mfma")
    assert w4.describe_dispatch(17, 12288, 1536, 256).startswith("mfma")
    set_dispatch_env(monkeypatch, W4_FORCE_PATH="")
    # group 32 below 5 rows, and K not a multiple of 128: vector ALU
    assert w4.describe_dispatch(4, 12288, 1536, 32).startswith("smallm MT=4")
    assert w4.describe_dispatch(8, 97, 288, 32).startswith("smallm MT=8")
    # activation rows within a CU's LDS: matrix cores; past it (16 x 6144
    # bf16 = 192 KB) the tiled kernel
    assert w4.describe_dispatch(8, 1536, 6144, 32).startswith("smallm mfma")
    assert w4.describe_dispatch(16, 1536, 2048, 32).startswith("smallm mfma")
    assert w4.describe_dispatch(16, 1536, 6144, 32).startswith("mfma")
    assert w4.describe_dispatch(33, 12288, 1536, 256).startswith("mfma")
    assert w4.describe_dispatch(64, 12288, 1536, 256).startswith("mfma")
    # DMA ring: block shape by workgroup rounds, K split for one-block grids,
    # up to 32 scale groups per row
    ring = lambda M, N, K, g: w4.describe_dispatch(M, N, K, g).split("block ")[1]
    assert ring(128, 12288, 1536, 256).startswith("64x64 waves 1x4")
    assert ring(320, 12288, 1536, 256).startswith("64x128 waves 1x4 slots 4")
    # three workgroups per CU (three-slot ring) where a round of them fits
    assert ring(384, 12288, 1536, 256).startswith("64x128 waves 1x4 slots 3")
    assert ring(512, 12288, 1536, 256).startswith("64x128 waves 1x4 slots 3")
    assert ring(640, 12288, 1536, 256).startswith("64x128 waves 1x4 slots 4")
    assert ring(1024, 12288, 1536, 256).startswith("64x128 waves 1x4 slots 3")
    assert ring(1984, 6336, 1536, 256).startswith("64x192 waves 1x4")  # fewer rounds
    assert ring(64, 1536, 6144, 256).startswith("64x64 waves 3x4")
    assert ring(256, 4096, 1536, 256).startswith("64x64 waves 3x4")
    assert ring(64, 1536, 8192, 256).startswith("64x64 waves 2x4")
    assert "dma-ring" not in w4.describe_dispatch(64, 1536, 1 << 14, 256)  # 64 groups
    assert ring(64, 12288, 1536, 32).startswith("64x64 waves 2x4")
    assert ring(128, 12288, 1536, 32).startswith("64x64 waves 1x4")
    assert ring(512, 12288, 1536, 32).startswith("64x128 waves 1x4 slots 3")
    assert ring(256, 12288, 1536, 32).startswith("64x128 waves 1x4 slots 4")
    assert ring(64, 1536, 6144, 32).startswith("64x64 waves 3x4")      # 192 groups
    assert ring(1024, 1536, 6144, 32).startswith("64x64 waves 2x4")
    assert "dma-ring" not in w4.describe_dispatch(64, 1536, 6400, 32)  # 200 groups
    with pytest.raises(w4.W4Error):
        w4.describe_dispatch(1, 12288, 1500, 32)


# ---------------------------------------------------------- host packer ---

def test_device_word_order_hand_typed(L):
    # canonical word 0x76543210 holds elements 0..7 = codes 0..7; the device
    # word keeps even elements (0, 2, 4, 6) in the low half-word and odd ones
    # (1, 3, 5, 7) in the high half-word, in order.
    cases = {0x76543210: 0x75316420, 0x88888888: 0x88888888,
             0xFEDCBA98: 0xFDB9ECA8, 0x0000000F: 0x0000000F,
             0x000000F0: 0x000F0000, 0xF0000000: 0xF0000000}
    for canon, dev in cases.items():
        P = np.array([[canon]], dtype=np.uint32)
        S = np.array([[0x3F80]], dtype=np.uint16)
        P4 = np.array([[canon, 0, 0, 0]], dtype=np.uint32)
        buf = w4.pack_host(P4, S, 1, 32, 32)
        assert int(buf[:4].view(np.uint32)[0]) == dev, hex(canon)
        assert int(buf[256:258].view(np.uint16)[0]) == 0x3F80


@pytest.mark.parametrize("N,K,group", [(1, 32, 32), (33, 96, 32), (7, 512, 256),
                                       (65, 1536, 32)])
def test_host_pack_round_trip(L, N, K, group):
    rng = np.random.default_rng(N * K)
    P, S = synth.draw_weights(rng, N, K, group)
    buf = w4.pack_host(P, S, N, K, group)
    assert buf.size == w4.packed_bytes(N, K, group)
    P2, S2 = w4.unpack_host(buf, N, K, group)
    assert np.array_equal(P, P2) and np.array_equal(S, S2)


def test_library_load_makes_no_gpu_call(L):
    # no device on this host: the build info is static, device_check fails cleanly
    assert "gfx950" in w4.build_info()
