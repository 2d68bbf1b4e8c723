"""The allocation-free entry point w4a16_gemm_noalloc, called through the
C ABI, against w4a16_gemm with a caller workspace: bitwise equal outputs on
two calls in a row (the second smaller), with and without the run-time
transform; a size beyond the static array is rejected before any launch."""
import numpy as np
import pytest

import bit_weight_only_w4a16_amd as w4
from bit_weight_only_w4a16_amd import synth

from _util import device, from_dev, note, to_dev_bf16, upload_packed

pytestmark = pytest.mark.gpu


def test_noalloc_matches_workspace_entry_point():
    import torch
    device()
    w4.device_check()
    N, K, g = 3072, 1536, 256
    rng = np.random.default_rng(71)
    P, S = synth.draw_weights(rng, N, K, g)
    packed = upload_packed(P, S, N, K, g)
    cap = w4.gemm_noalloc_max_bytes()
    assert cap == 8 << 20
    # two calls in a row, the second smaller; the transform and the plain
    # product; several row counts so that every dispatch path is covered
    for M, had in ((512, 512), (96, 512), (64, 0), (8, 512), (3, 512), (1, 512)):
        X = to_dev_bf16(synth.draw_activations(rng, M, K, outlier_frac=0.01))
        note("noalloc gemm M=%d had=%d" % (M, had))
        for odt in ("bf16", "f32"):
            ref = from_dev(w4.gemm(packed, N, K, g, X, had_block=had, out_dtype=odt))
            got = from_dev(w4.gemm_noalloc(packed, N, K, g, X, had_block=had, out_dtype=odt))
            torch.cuda.synchronize()
            assert np.array_equal(ref.view(np.uint32) if odt == "f32" else ref, got.view(
                np.uint32) if odt == "f32" else got), (M, had, odt)


def test_noalloc_rejects_oversize():
    device()
    N, K, g = 64, 4096, 256
    rng = np.random.default_rng(3)
    P, S = synth.draw_weights(rng, N, K, g)
    packed = upload_packed(P, S, N, K, g)
    M = (8 << 20) // (K * 2) + 1
    X = to_dev_bf16(synth.draw_activations(rng, M, K))
    with pytest.raises(w4.W4Error) as e:
        w4.gemm_noalloc(packed, N, K, g, X, had_block=512)
    assert e.value.status == -2
    # the plain product needs no scratch and is accepted at that size
    w4.gemm_noalloc(packed, N, K, g, X, had_block=0)
