"""w4_gemv_noalloc: the GEMV entry point that allocates nothing.

Its split-K partials live in the library's fixed per-device scratch instead
of a caller workspace; the kernels and plan are w4_gemv's, so its outputs
must be bit-identical to w4_gemv's.  Two calls in a row, the second smaller,
exercise the reuse of the scratch (the second call's partials overwrite a
prefix of the first's), and a third needs no scratch at all.  A shape whose
partials exceed the scratch is refused on the host."""
import ctypes
import os

import numpy as np
import pytest
import torch

import bit_weight_quantized_amd as w4
import workloads as wl
from gpu_helpers import announce, dev, host, require_gpu

W4_EWORKSPACE = -3
SCRATCH_BYTES = 4 << 20


def weights(K, N, G, fmt, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    w = torch.randn((N, K), generator=gen, device="cuda", dtype=torch.float32) * 0.02
    codes, scale, zero = w4.quantize(w, G, fmt)
    return w4.pack(codes), scale, zero


@pytest.mark.gpu
def test_noalloc_matches_gemv_on_consecutive_calls():
    require_gpu()
    cases = [(32, 28672, 8192, 0, 128), (1, 8192, 1024, 1, 64), (4, 8192, 8192, 0, 128)]
    plans = [w4.gemv_plan(M, K, N, G, fmt) for M, K, N, fmt, G in cases]
    assert plans[0]["workspace_bytes"] == SCRATCH_BYTES      # the whole scratch
    assert 0 < plans[1]["workspace_bytes"] < SCRATCH_BYTES   # a prefix of it
    assert plans[2]["workspace_bytes"] == 0                  # no split K
    for i, (M, K, N, fmt, G) in enumerate(cases):
        packed, scale, zero = weights(K, N, G, fmt, 900 + i)
        x = dev(wl.make_activations(3 if K == 28672 else 2, i, M, K))
        announce("gemv_noalloc", dict(M=M, K=K, N=N, fmt=fmt, G=G))
        y_ref = host(w4.gemv(x, packed, scale, zero, G, fmt))
        y1 = host(w4.gemv_noalloc(x, packed, scale, zero, G, fmt))
        torch.cuda.synchronize()
        assert np.array_equal(y1.view(np.uint16), y_ref.view(np.uint16)), (M, K, N, fmt)
        assert np.isfinite(y1.astype(np.float32)).all()


def test_noalloc_refuses_shapes_beyond_the_scratch():
    """Host-side refusal before anything is enqueued (no GPU needed: the
    pointers are never dereferenced)."""
    if not os.path.exists(w4.lib_path):
        import bit_weight_quantized_amd.build as b
        b.build()
    L = w4.lib()
    fake = ctypes.c_void_p(0x7F0000001000)
    M, K, N, G = 32, 32768, 16384, 128
    assert w4.gemv_plan(M, K, N, G, 0)["workspace_bytes"] > SCRATCH_BYTES
    st = L.w4_gemv_noalloc(fake, M, K, N, fake, fake, fake, G, 0, fake, None)
    assert st == W4_EWORKSPACE
    assert b"scratch" in L.w4_last_error()
    # the same rules as w4_gemv otherwise
    assert L.w4_gemv_noalloc(fake, 33, 256, 32, fake, fake, fake, 128, 0, fake, None) == -1
    assert L.w4_gemv_noalloc(fake, 1, 256, 32, fake, fake, None, 128, 0, fake, None) == -1
