"""Host-only checks of the C ABI (no GPU needed, no compute launched).

* libw4.so loads and exports every function include/w4.h declares;
* the library's NF4 level table is bit-equal to the oracle's derivation;
* argument errors return their documented status before anything is enqueued.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as o

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4.h")

W4_OK, W4_EINVAL, W4_EUNSUPPORTED, W4_EWORKSPACE, W4_EHIP = 0, -1, -2, -3, -4


@pytest.fixture(scope="module")
def L():
    import bit_weight_quantized_amd as w4
    if not os.path.exists(w4.lib_path):
        import bit_weight_quantized_amd.build as b
        b.build()
    return w4.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    fns = declared_functions()
    for want in ("w4_quantize", "w4_pack", "w4_gemv", "w4_gemm", "w4_gemm_decomp",
                 "w4_gemm_decomp_fixed", "w4_workspace_bytes", "w4_status_str", "w4_last_error"):
        assert want in fns


def test_library_exports_every_declared_symbol(L):
    missing = [f for f in declared_functions() if not hasattr(L, f)]
    assert not missing, missing


def test_nf4_levels_bit_equal_to_oracle(L):
    import bit_weight_quantized_amd as w4
    lib_levels = np.array(w4.nf4_levels(), dtype=np.float32)
    assert np.array_equal(lib_levels.view(np.uint32), o.nf4_codebook().view(np.uint32))


def test_status_strings(L):
    for st in (W4_OK, W4_EINVAL, W4_EUNSUPPORTED, W4_EWORKSPACE, W4_EHIP):
        assert L.w4_status_str(st)
    assert L.w4_version().startswith(b"w4")


FAKE = ctypes.c_void_p(0x7F0000001000)  # never dereferenced: every call below fails validation first
MISALIGNED = ctypes.c_void_p(0x7F0000001001)


def _gemv(L, M=1, K=256, N=32, packed=FAKE, scale=FAKE, zero=FAKE, G=128, fmt=0, x=FAKE, y=FAKE):
    return L.w4_gemv(x, M, K, N, packed, scale, zero, G, fmt, y, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=0), W4_EINVAL),
    (dict(M=33), W4_EINVAL),
    (dict(K=200), W4_EINVAL),          # K % G != 0
    (dict(K=192, G=64), W4_EINVAL),    # K % 128 != 0 (the weight tile)
    (dict(G=32, K=256), W4_EINVAL),    # G not in {64, 128}
    (dict(N=40), W4_EINVAL),           # N % 16 != 0
    (dict(fmt=7), W4_EINVAL),
    (dict(zero=None), W4_EINVAL),      # INT4 without zero points
    (dict(fmt=1), W4_EINVAL),          # NF4 with zero points
    (dict(x=None), W4_EINVAL),
    (dict(packed=MISALIGNED), W4_EINVAL),
])
def test_gemv_argument_errors(L, kw, status):
    assert _gemv(L, **kw) == status
    assert L.w4_last_error()  # a message was recorded


def test_gemm_argument_errors(L):
    args = [FAKE, 64, 256, 32, FAKE, FAKE, FAKE, 128, 0]
    assert L.w4_gemm(*args, 5, FAKE, None, 0, None) == W4_EINVAL  # unknown mode
    assert L.w4_gemm(FAKE, 64, 256, 30, FAKE, FAKE, FAKE, 128, 0, 0, FAKE, None, 0, None) == W4_EINVAL


def test_decomp_argument_errors(L):
    base = dict(x=FAKE, M=4, K=256, N=32, packed=FAKE, scale=FAKE, zero=FAKE, G=128, ns=2)

    def call(**kw):
        a = {**base, **kw}
        return L.w4_gemm_decomp(a["x"], a["M"], a["K"], a["N"], a["packed"], a["scale"], a["zero"],
                                a["G"], a["ns"], FAKE, None, None, None, a.get("ws"),
                                a.get("wsb", 0), None)
    assert call(ns=4) == W4_EINVAL
    assert call(ns=0) == W4_EINVAL
    assert call(ns=3) == W4_EWORKSPACE  # three slices are valid; still no workspace
    assert call(zero=None) == W4_EUNSUPPORTED  # NF4 weights cannot feed int8 matrix cores
    assert call() == W4_EWORKSPACE              # slices/scales need a workspace
    need = L.w4_workspace_bytes(4, 4, 256, 32, 128, 2)
    assert need >= 2 * 4 * 256 + 2 * 4 * 4
    assert call(ws=FAKE, wsb=need - 1) == W4_EWORKSPACE


def test_decomp_fixed_argument_errors(L):
    base = dict(x=FAKE, M=4, K=256, N=32, packed=FAKE, scale=FAKE, zero=FAKE, G=128)

    def call(**kw):
        a = {**base, **kw}
        return L.w4_gemm_decomp_fixed(a["x"], a["M"], a["K"], a["N"], a["packed"], a["scale"], a["zero"],
                                      a["G"], FAKE, None, None, None, a.get("ws"), a.get("wsb", 0), None)
    assert call(zero=None) == W4_EUNSUPPORTED
    assert call(G=32) == W4_EINVAL
    assert call(N=40) == W4_EINVAL
    assert call() == W4_EWORKSPACE
    need = L.w4_workspace_bytes(4, 4, 256, 32, 128, 2)
    assert call(ws=FAKE, wsb=need - 1) == W4_EWORKSPACE
    assert call(ws=MISALIGNED, wsb=need) == W4_EINVAL
    assert b"w4_gemm_decomp_fixed" in L.w4_last_error()


def test_decomp_fixed_fused_argument_errors(L):
    base = dict(x=FAKE, M=4, K=256, N=32, packed=FAKE, scale=FAKE, zero=FAKE, G=128)

    def call(**kw):
        a = {**base, **kw}
        return L.w4_gemm_decomp_fixed_fused(a["x"], a["M"], a["K"], a["N"], a["packed"], a["scale"], a["zero"],
                                            a["G"], FAKE, a.get("ts"), a.get("ws"), a.get("wsb", 0), None)
    assert call(zero=None) == W4_EUNSUPPORTED
    assert call(G=32) == W4_EINVAL
    assert call(K=192, G=64) == W4_EINVAL  # not a multiple of the 128-position tile
    assert call(N=40) == W4_EINVAL
    assert call(M=0) == W4_EINVAL
    assert call() == W4_EWORKSPACE
    need = L.w4_workspace_bytes(7, 4, 256, 0, 128, 0)
    assert need == 256  # fp32 token scales [2][4], 256-byte aligned
    assert call(ws=FAKE, wsb=need - 1) == W4_EWORKSPACE
    assert call(ws=MISALIGNED, wsb=need) == W4_EINVAL
    assert call(ts=MISALIGNED, ws=FAKE, wsb=need) == W4_EINVAL
    assert b"w4_gemm_decomp_fixed_fused" in L.w4_last_error()
    # with the real N the workspace adds the tail partials of the fixed-ratio product's plan
    assert L.w4_workspace_bytes(7, 300, 1024, 4096, 128, 0) >= need
    assert L.w4_workspace_bytes(7, 4, 192, 32, 64, 0) == 256 and L.w4_workspace_bytes(7, 4, 200, 32, 64, 0) == 0


def test_stream_read_argument_errors(L):
    assert L.w4_stream_read(FAKE, 24, FAKE, None) == W4_EINVAL  # not whole 16-byte pieces
    assert L.w4_stream_read(None, 32, FAKE, None) == W4_EINVAL
    assert L.w4_stream_read(FAKE, 32, None, None) == W4_EINVAL
    assert L.w4_stream_read(MISALIGNED, 32, FAKE, None) == W4_EINVAL
    assert b"w4_stream_read" in L.w4_last_error()
    assert L.w4_stream_read(None, 0, None, None) == W4_OK  # nothing to read


def test_residual_argument_errors(L):
    # selection: K beyond the LDS-resident key array, k beyond K or 1024, nulls
    assert L.w4_salient_select(FAKE, 1, 32769, 4, FAKE, None) == W4_EINVAL
    assert L.w4_salient_select(FAKE, 1, 100, 101, FAKE, None) == W4_EINVAL
    assert L.w4_salient_select(FAKE, 1, 4096, 1025, FAKE, None) == W4_EINVAL
    assert L.w4_salient_select(FAKE, 0, 100, 4, FAKE, None) == W4_EINVAL
    assert L.w4_salient_select(None, 1, 100, 4, FAKE, None) == W4_EINVAL
    assert L.w4_salient_select(FAKE, 1, 100, 0, None, None) == W4_OK  # k = 0: nothing to do
    # correction: M in 1..32, N % 8, operands, alignment
    args = dict(x=FAKE, M=1, K=64, N=64, r=FAKE, idx=FAKE, k=4, y=FAKE)

    def corr(**kw):
        a = {**args, **kw}
        return L.w4_residual_correct(a["x"], a["M"], a["K"], a["N"], a["r"], a["idx"], a["k"], a["y"], None)
    assert corr(M=33) == W4_EINVAL
    assert corr(N=12) == W4_EINVAL
    assert corr(k=-1) == W4_EINVAL
    assert corr(r=None) == W4_EINVAL
    assert corr(idx=None) == W4_EINVAL
    assert corr(r=MISALIGNED) == W4_EINVAL
    assert b"w4_residual_correct" in L.w4_last_error()
    # selection and correction in one launch: both sets of bounds

    def sc(**kw):
        a = {**args, **kw}
        return L.w4_salient_correct(a["x"], a["M"], a["K"], a["N"], a["r"], a["k"], a["idx"], a["y"], None)
    assert sc(M=33) == W4_EINVAL
    assert sc(K=32769) == W4_EINVAL
    assert sc(N=12) == W4_EINVAL
    assert sc(k=65) == W4_EINVAL  # k > K
    assert sc(K=4096, k=1025) == W4_EINVAL
    assert sc(k=-1) == W4_EINVAL
    assert sc(r=None) == W4_EINVAL
    assert sc(idx=None) == W4_EINVAL
    assert sc(y=MISALIGNED) == W4_EINVAL
    assert b"w4_salient_correct" in L.w4_last_error()
    # the correction stored in fp32, and its application to y

    def c32(**kw):
        a = {**args, **kw}
        return L.w4_residual_correct_f32(a["x"], a["M"], a["K"], a["N"], a["r"], a["idx"], a["k"], a["y"], None)
    assert c32(M=0) == W4_EINVAL
    assert c32(M=33) == W4_EINVAL
    assert c32(N=12) == W4_EINVAL
    assert c32(k=-1) == W4_EINVAL
    assert c32(y=None) == W4_EINVAL
    assert c32(idx=None) == W4_EINVAL
    assert c32(y=MISALIGNED) == W4_EINVAL
    assert b"w4_residual_correct_f32" in L.w4_last_error()
    assert L.w4_residual_apply(FAKE, 0, 64, FAKE, None) == W4_EINVAL
    assert L.w4_residual_apply(FAKE, 1, 12, FAKE, None) == W4_EINVAL
    assert L.w4_residual_apply(None, 1, 64, FAKE, None) == W4_EINVAL
    assert L.w4_residual_apply(FAKE, 1, 64, MISALIGNED, None) == W4_EINVAL
    assert b"w4_residual_apply" in L.w4_last_error()

    def sc32(**kw):
        a = {**args, **kw}
        return L.w4_salient_correct_f32(a["x"], a["M"], a["K"], a["N"], a["r"], a["k"], a["idx"], a["y"], None)
    assert sc32(M=33) == W4_EINVAL
    assert sc32(K=32769) == W4_EINVAL
    assert sc32(N=12) == W4_EINVAL
    assert sc32(k=65) == W4_EINVAL  # k > K
    assert sc32(K=4096, k=1025) == W4_EINVAL
    assert sc32(k=-1) == W4_EINVAL
    assert sc32(y=None) == W4_EINVAL
    assert sc32(idx=None) == W4_EINVAL
    assert sc32(y=MISALIGNED) == W4_EINVAL
    assert b"w4_salient_correct_f32" in L.w4_last_error()


def test_mx_argument_errors(L):
    assert L.w4_quantize_mx(FAKE, 100, 16, FAKE, FAKE, None) == W4_EINVAL   # K % 32
    assert L.w4_quantize_mx(None, 128, 16, FAKE, FAKE, None) == W4_EINVAL
    assert L.w4_pack_mx(FAKE, 96, 16, FAKE, None) == W4_EINVAL             # K % 128
    assert L.w4_pack_mx(FAKE, 128, 24, FAKE, None) == W4_EINVAL            # N % 16
    assert L.w4_pack_mx(FAKE, 128, 16, MISALIGNED, None) == W4_EINVAL

    def g(M=4, K=256, N=32, ns=2, ws=None, wsb=0, x=FAKE):
        return L.w4_gemm_mx(x, M, K, N, FAKE, FAKE, ns, FAKE, None, None, ws, wsb, None)
    assert g(ns=3) == W4_EINVAL
    assert g(K=192) == W4_EINVAL
    assert g(N=24) == W4_EINVAL
    assert g(M=0) == W4_EINVAL
    assert g(x=MISALIGNED) == W4_EINVAL
    assert g() == W4_EWORKSPACE
    need = L.w4_workspace_bytes(5, 4, 256, 32, 32, 2)
    assert need == 1024 + 256  # slices 2*4*128 bytes, scales 2*4*8 bytes rounded up to 256
    assert g(ws=FAKE, wsb=need - 1) == W4_EWORKSPACE
    assert L.w4_workspace_bytes(5, 4, 256, 32, 32, 3) == 0


def test_attn_argument_errors(L):
    def a(B=1, Hq=8, Hkv=1, Lp=256, d=128, ws=None, wsb=0, q=FAKE):
        return L.w4_attn_decode_msd(q, B, Hq, Hkv, Lp, d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, wsb, None)
    assert a(d=64) == W4_EUNSUPPORTED
    assert a(Hq=8, Hkv=3) == W4_EINVAL
    assert a(Hq=34, Hkv=2) == W4_EINVAL   # 17 query heads per kv head
    assert a(Lp=300) == W4_EINVAL
    assert a(q=None) == W4_EINVAL
    assert a() == W4_EWORKSPACE
    need = L.w4_workspace_bytes(6, 1, 8, 256, 0, 0)
    assert need > 8 * 128 * 4  # at least the partial outputs
    assert a(ws=FAKE, wsb=need - 1) == W4_EWORKSPACE


def test_quantize_and_pack_argument_errors(L):
    assert L.w4_quantize(FAKE, 100, 16, 64, 0, FAKE, FAKE, FAKE, None) == W4_EINVAL
    assert L.w4_quantize(FAKE, 128, 16, 64, 1, FAKE, FAKE, FAKE, None) == W4_EINVAL  # NF4 + zero
    assert L.w4_quantize(FAKE, 128, 16, 64, 0, FAKE, FAKE, None, None) == W4_EINVAL  # INT4 no zero
    assert L.w4_pack(FAKE, 48, 16, FAKE, None) == W4_EINVAL
    assert L.w4_pack(MISALIGNED, 128, 16, FAKE, None) == W4_EINVAL
    assert L.w4_pack(FAKE, 192, 16, FAKE, None) == W4_EINVAL   # K % 128 != 0 (the weight tile)
    assert L.w4_pack(FAKE, 128, 24, FAKE, None) == W4_EINVAL   # N % 16 != 0


def test_workspace_bytes(L):
    assert L.w4_workspace_bytes(2, 1, 8192, 8192, 128, 0) == 0
    # decomposition: slices [nslices][M][K] then fp32 scales [nslices][M], each 256-byte aligned
    for ns in (1, 2, 3):
        want = -(-ns * 100 * 1024 // 256) * 256 + -(-ns * 100 * 4 // 256) * 256
        assert L.w4_workspace_bytes(4, 100, 1024, 64, 128, ns) == want
    assert L.w4_workspace_bytes(4, 100, 1024, 64, 128, 4) == 0
    assert L.w4_workspace_bytes(99, 1, 1, 1, 1, 0) == ctypes.c_size_t(-1).value


def test_mfma_rate_argument_errors(L):
    assert L.w4_mfma_rate(2, 0, 1, 1, FAKE, None, None) == W4_EINVAL  # kind
    assert L.w4_mfma_rate(0, 5, 1, 1, FAKE, None, None) == W4_EINVAL  # valu not instantiated
    assert L.w4_mfma_rate(0, 9, 1, 1, FAKE, None, None) == W4_EINVAL
    assert L.w4_mfma_rate(1, 0, 0, 1, FAKE, None, None) == W4_EINVAL  # no workgroups
    assert L.w4_mfma_rate(1, 0, 1, 0, FAKE, None, None) == W4_EINVAL  # no iterations
    assert L.w4_mfma_rate(0, 0, 1, 1, None, None, None) == W4_EINVAL  # sink
    assert L.w4_mfma_rate(0, 0, 1, 1, MISALIGNED, None, None) == W4_EINVAL
    assert b"w4_mfma_rate" in L.w4_last_error()
