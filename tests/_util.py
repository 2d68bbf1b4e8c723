"""Helpers for the GPU parity tests: device uploads and the acceptance rule.

Acceptance (per output element, against the fp64 oracle):
    |y_gpu - y| <= 2e-3 * sum_k |w_k x_k|            (fp32 output)
    |y_gpu - y| <= 2e-3 * sum_k |w_k x_k| + ulp(y)    (bf16 output)
with ulp(y) = 2^(floor(log2 |y|) - 7) the spacing of bf16 numbers at y
(0 when y == 0).  Dequantized values are checked bit-exactly separately.
"""
import sys

import numpy as np


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    return torch.device("cuda:0")


def to_dev_u32(a):
    import torch
    a = np.ascontiguousarray(a, dtype=np.uint32)
    return torch.from_numpy(a.view(np.int32)).to(device())


def to_dev_bf16(a):
    import torch
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).to(device()).view(torch.bfloat16)


def to_dev_u16(a):
    import torch
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).to(device())


def from_dev(t):
    """float32 numpy array of a float32 or bfloat16 device tensor (exact)."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy()


def bf16_ulp(y):
    y = np.abs(np.asarray(y, dtype=np.float64))
    out = np.zeros_like(y)
    nz = y > 0
    out[nz] = np.exp2(np.floor(np.log2(y[nz])) - 7)
    return out


def bound(Y, A, out_dtype):
    b = 2e-3 * np.asarray(A, dtype=np.float64)
    if out_dtype == "bf16":
        b = b + bf16_ulp(Y)
    return b


def assert_within(got, Y, A, out_dtype, what=""):
    got = np.asarray(got, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    err = np.abs(got - Y)
    b = bound(Y, A, out_dtype)
    bad = err > b
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            "%s: %d of %d outputs out of tolerance; first %s: got %s want %s bound %s"
            % (what, int(bad.sum()), bad.size, idx.tolist(),
               got[tuple(idx.T)].tolist(), Y[tuple(idx.T)].tolist(),
               b[tuple(idx.T)].tolist()))
    return float((err / np.maximum(b, 1e-300)).max())


def upload_packed(case_P, case_S, N, K, group):
    """Canonical arrays -> device, packed on the device by w4_pack."""
    import bit_weight_only_w4a16_amd as w4
    P = to_dev_u32(case_P)
    S = to_dev_u16(case_S)
    packed = w4.pack(P, S, N, K, group)
    return packed


def set_dispatch_env(monkeypatch, **env):
    """Set W4_* dispatch variables for this test and make the library re-read
    them (the conftest fixture restores the configuration afterwards)."""
    import bit_weight_only_w4a16_amd as w4
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    w4.config_reload()
