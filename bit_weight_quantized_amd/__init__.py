"""Python binding of libw4.so, the gfx950 4-bit weight-quantized matmul library.

Argument marshalling only: every step of the computation runs in the HIP
library.  PyTorch provides device memory and the current HIP stream.  The
functions take and return torch tensors on the GPU; fp16 data are
``torch.float16`` tensors whose bits travel through the C ABI as uint16.

Entry points mirror ``include/w4.h``: quantize, pack, gemv, gemm,
gemm_decomp, workspace_bytes, nf4_levels.  If the library is not built,
importing works but the first call raises ``W4LibraryMissing``; nothing
falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "INT4_ASYM", "NF4", "DQ_F16", "POSTSCALE", "W4Error", "W4LibraryMissing",
    "lib", "lib_path", "quantize", "pack", "gemv", "gemv_noalloc", "gemv_plan", "gemm", "gemm_decomp", "gemm_decomp_fixed",
    "gemm_decomp_fixed_fused", "stream_read", "mfma_rate",
    "salient_select", "residual_correct", "salient_correct", "residual_correct_f32", "residual_apply",
    "salient_correct_f32", "quantize_mx", "pack_mx", "gemm_mx", "attn_decode_msd",
    "workspace_bytes", "nf4_levels", "version",
]

INT4_ASYM = 0
NF4 = 1
DQ_F16 = 0
POSTSCALE = 1
STREAM_READ_ACC_WORDS = 449  # W4_STREAM_READ_ACC_WORDS
OP_QUANTIZE, OP_PACK, OP_GEMV, OP_GEMM, OP_GEMM_DECOMP, OP_GEMM_MX, OP_ATTN_MSD, OP_GEMM_DECOMP_FUSED = range(8)

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libw4.so")
_lib = None

_p = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t


class W4LibraryMissing(RuntimeError):
    pass


class W4Error(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib():
    """Load libw4.so (once) and declare its C signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise W4LibraryMissing(
                f"{lib_path} is not built; run `python -m bit_weight_quantized_amd.build` "
                "or __graft_entry__.build()")
        L = ctypes.CDLL(lib_path)
        L.w4_quantize.argtypes = [_p, _i, _i, _i, _i, _p, _p, _p, _p]
        L.w4_pack.argtypes = [_p, _i, _i, _p, _p]
        L.w4_gemv.argtypes = [_p, _i, _i, _i, _p, _p, _p, _i, _i, _p, _p, _sz, _p]
        L.w4_gemv_plan.argtypes = [_i, _i, _i, _i, _i, _p, _i]
        L.w4_gemv_noalloc.argtypes = [_p, _i, _i, _i, _p, _p, _p, _i, _i, _p, _p]
        L.w4_gemm.argtypes = [_p, _i, _i, _i, _p, _p, _p, _i, _i, _i, _p, _p, _sz, _p]
        L.w4_gemm_decomp.argtypes = [_p, _i, _i, _i, _p, _p, _p, _i, _i, _p, _p, _p, _p, _p, _sz, _p]
        L.w4_gemm_decomp_fixed.argtypes = [_p, _i, _i, _i, _p, _p, _p, _i, _p, _p, _p, _p, _p, _sz, _p]
        L.w4_gemm_decomp_fixed_fused.argtypes = [_p, _i, _i, _i, _p, _p, _p, _i, _p, _p, _p, _sz, _p]
        L.w4_stream_read.argtypes = [_p, _sz, _p, _p]
        L.w4_mfma_rate.argtypes = [_i, _i, _i, _i, _p, _p, _p]
        L.w4_salient_select.argtypes = [_p, _i, _i, _i, _p, _p]
        L.w4_quantize_mx.argtypes = [_p, _i, _i, _p, _p, _p]
        L.w4_pack_mx.argtypes = [_p, _i, _i, _p, _p]
        L.w4_gemm_mx.argtypes = [_p, _i, _i, _i, _p, _p, _i, _p, _p, _p, _p, _sz, _p]
        L.w4_attn_decode_msd.argtypes = [_p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]
        L.w4_residual_correct.argtypes = [_p, _i, _i, _i, _p, _p, _i, _p, _p]
        L.w4_salient_correct.argtypes = [_p, _i, _i, _i, _p, _i, _p, _p, _p]
        L.w4_residual_correct_f32.argtypes = [_p, _i, _i, _i, _p, _p, _i, _p, _p]
        L.w4_residual_apply.argtypes = [_p, _i, _i, _p, _p]
        L.w4_salient_correct_f32.argtypes = [_p, _i, _i, _i, _p, _i, _p, _p, _p]
        L.w4_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i]
        L.w4_workspace_bytes.restype = _sz
        L.w4_nf4_levels.argtypes = [_p]
        L.w4_status_str.argtypes = [_i]
        L.w4_status_str.restype = ctypes.c_char_p
        L.w4_last_error.argtypes = []
        L.w4_last_error.restype = ctypes.c_char_p
        L.w4_version.restype = ctypes.c_char_p
        for fn in ("w4_quantize", "w4_pack", "w4_gemv", "w4_gemv_noalloc", "w4_gemv_plan", "w4_gemm", "w4_gemm_decomp", "w4_gemm_decomp_fixed",
                   "w4_gemm_decomp_fixed_fused", "w4_stream_read", "w4_mfma_rate", "w4_salient_select", "w4_residual_correct", "w4_salient_correct",
                   "w4_residual_correct_f32", "w4_residual_apply", "w4_salient_correct_f32", "w4_quantize_mx", "w4_pack_mx", "w4_gemm_mx",
                   "w4_attn_decode_msd",
                   "w4_nf4_levels"):
            getattr(L, fn).restype = _i
        _lib = L
    return _lib


def _check(fn, status):
    if status != 0:
        raise W4Error(fn, status, lib().w4_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, dtype, name):
    if not (t.is_cuda and t.dtype == dtype and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor")
    return t


def version() -> str:
    return lib().w4_version().decode()


def nf4_levels() -> "list[float]":
    """The library's 16 fp32 NF4 levels (host copy)."""
    buf = (ctypes.c_float * 16)()
    _check("w4_nf4_levels", lib().w4_nf4_levels(ctypes.cast(buf, _p)))
    return list(buf)


def workspace_bytes(op: int, M: int, K: int, N: int, G: int, fmt_or_mode: int) -> int:
    return int(lib().w4_workspace_bytes(op, M, K, N, G, fmt_or_mode))


def quantize(wt, G: int, fmt: int, *, codes=None, scale=None, zero=None, stream=None):
    """Quantize fp32 W^T [N][K] -> (codes uint8 [N][K], scale fp16 [N][K/G],
    zero fp16 [N][K/G] or None for NF4)."""
    _dev(wt, torch.float32, "wt")
    N, K = wt.shape
    codes = torch.empty((N, K), dtype=torch.uint8, device=wt.device) if codes is None else codes
    ng = K // G if G else 0
    scale = torch.empty((N, ng), dtype=torch.float16, device=wt.device) if scale is None else scale
    if fmt == INT4_ASYM and zero is None:
        zero = torch.empty((N, ng), dtype=torch.float16, device=wt.device)
    _check("w4_quantize", lib().w4_quantize(_ptr(wt), K, N, G, fmt, _ptr(codes), _ptr(scale),
                                            _ptr(zero) if fmt == INT4_ASYM else None, _stream(stream)))
    return codes, scale, (zero if fmt == INT4_ASYM else None)


def pack(codes, *, out=None, stream=None):
    """Pack codes [N][K] -> [N][K/2] bytes (low nibble = even k)."""
    _dev(codes, torch.uint8, "codes")
    N, K = codes.shape
    out = torch.empty((N, K // 2), dtype=torch.uint8, device=codes.device) if out is None else out
    _check("w4_pack", lib().w4_pack(_ptr(codes), K, N, _ptr(out), _stream(stream)))
    return out


def _weights(packed, scale, zero):
    _dev(packed, torch.uint8, "packed")
    _dev(scale, torch.float16, "scale")
    if zero is not None:
        _dev(zero, torch.float16, "zero")
    N, half_k = packed.shape
    return N, 2 * half_k


def gemv(x, packed, scale, zero, G: int, fmt: int, *, out=None, workspace=None, stream=None):
    """y[M][N] = x[M][K] . W' for 1 <= M <= 32 (fp16 in, fp16 out)."""
    _dev(x, torch.float16, "x")
    N, K = _weights(packed, scale, zero)
    M = x.shape[0]
    out = torch.empty((M, N), dtype=torch.float16, device=x.device) if out is None else out
    ws_n = workspace_bytes(OP_GEMV, M, K, N, G, fmt)
    if workspace is None and ws_n:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=x.device)
    _check("w4_gemv", lib().w4_gemv(_ptr(x), M, K, N, _ptr(packed), _ptr(scale), _ptr(zero), G, fmt,
                                    _ptr(out), _ptr(workspace),
                                    0 if workspace is None else workspace.numel(), _stream(stream)))
    return out


def gemv_noalloc(x, packed, scale, zero, G: int, fmt: int, *, out=None, stream=None):
    """w4_gemv without a workspace: split-K partials in the library's fixed
    per-device scratch (calls on one device must not overlap in time)."""
    _dev(x, torch.float16, "x")
    N, K = _weights(packed, scale, zero)
    M = x.shape[0]
    out = torch.empty((M, N), dtype=torch.float16, device=x.device) if out is None else out
    _check("w4_gemv_noalloc", lib().w4_gemv_noalloc(_ptr(x), M, K, N, _ptr(packed), _ptr(scale), _ptr(zero), G,
                                                    fmt, _ptr(out), _stream(stream)))
    return out


GEMV_PLAN_FIELDS = ("kernel", "cols", "token_tiles", "row_waves", "k_waves", "k_slices", "staged_units",
                    "workgroups", "threads", "lds_bytes", "lds_budget", "static_lds", "workspace_bytes", "ok",
                    "ring", "act_lds")


def gemv_plan(M: int, K: int, N: int, G: int, fmt: int) -> dict:
    """The launch plan w4_gemv would use for this shape (host only; the
    W4_GEMV_* environment overrides of this process apply)."""
    buf = (ctypes.c_int64 * len(GEMV_PLAN_FIELDS))()
    _check("w4_gemv_plan", lib().w4_gemv_plan(M, K, N, G, fmt, ctypes.cast(buf, _p), len(GEMV_PLAN_FIELDS)))
    return dict(zip(GEMV_PLAN_FIELDS, (int(v) for v in buf)))


def gemm(x, packed, scale, zero, G: int, fmt: int, mode: int, *, out=None, workspace=None, stream=None):
    """y[M][N] = x[M][K] . W' on fp16 matrix cores, mode DQ_F16 or POSTSCALE."""
    _dev(x, torch.float16, "x")
    N, K = _weights(packed, scale, zero)
    M = x.shape[0]
    out = torch.empty((M, N), dtype=torch.float16, device=x.device) if out is None else out
    ws_n = workspace_bytes(OP_GEMM, M, K, N, G, mode)
    if workspace is None and ws_n:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=x.device)
    _check("w4_gemm", lib().w4_gemm(_ptr(x), M, K, N, _ptr(packed), _ptr(scale), _ptr(zero), G, fmt,
                                    mode, _ptr(out), _ptr(workspace),
                                    0 if workspace is None else workspace.numel(), _stream(stream)))
    return out


def gemm_decomp(x, packed, scale, zero, G: int, nslices: int = 2, *, out=None, slices_out=None,
                tok_scale_out=None, acc_out=None, workspace=None, stream=None):
    """Multi-Scale Dequant product: x split into int8 slices, int8 matrix cores.

    Returns y, or (y, slices, tok_scales, acc) when any optional output is
    given (pass tensors to receive them)."""
    _dev(x, torch.float16, "x")
    N, K = _weights(packed, scale, zero)
    M = x.shape[0]
    out = torch.empty((M, N), dtype=torch.float16, device=x.device) if out is None else out
    ws_n = workspace_bytes(OP_GEMM_DECOMP, M, K, N, G, nslices)
    if workspace is None and ws_n:  # slices, scales (unless given) and per-group slice sums
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=x.device)
    _check("w4_gemm_decomp", lib().w4_gemm_decomp(
        _ptr(x), M, K, N, _ptr(packed), _ptr(scale), _ptr(zero), G, nslices, _ptr(out),
        _ptr(slices_out), _ptr(tok_scale_out), _ptr(acc_out), _ptr(workspace),
        0 if workspace is None else workspace.numel(), _stream(stream)))
    if slices_out is None and tok_scale_out is None and acc_out is None:
        return out
    return out, slices_out, tok_scale_out, acc_out


def gemm_decomp_fixed(x, packed, scale, zero, G: int, *, out=None, slices_out=None,
                      tok_scale_out=None, acc_out=None, workspace=None, stream=None):
    """Two-slice Multi-Scale Dequant product with s_2 = s_1 / 254: the two int8
    products combine exactly in integers.  Returns as ``gemm_decomp``."""
    _dev(x, torch.float16, "x")
    N, K = _weights(packed, scale, zero)
    M = x.shape[0]
    out = torch.empty((M, N), dtype=torch.float16, device=x.device) if out is None else out
    ws_n = workspace_bytes(OP_GEMM_DECOMP, M, K, N, G, 2)
    if workspace is None and ws_n:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=x.device)
    _check("w4_gemm_decomp_fixed", lib().w4_gemm_decomp_fixed(
        _ptr(x), M, K, N, _ptr(packed), _ptr(scale), _ptr(zero), G, _ptr(out),
        _ptr(slices_out), _ptr(tok_scale_out), _ptr(acc_out), _ptr(workspace),
        0 if workspace is None else workspace.numel(), _stream(stream)))
    if slices_out is None and tok_scale_out is None and acc_out is None:
        return out
    return out, slices_out, tok_scale_out, acc_out


def gemm_decomp_fixed_fused(x, packed, scale, zero, G: int, *, out=None, tok_scale_out=None, workspace=None,
                            stream=None):
    """The fixed-ratio Multi-Scale Dequant product with the decomposition
    inside the product's K loop (only the token scales are computed first);
    y equals ``gemm_decomp_fixed``'s bit for bit.  Returns y, or
    (y, tok_scale_out) when tok_scale_out is given."""
    _dev(x, torch.float16, "x")
    N, K = _weights(packed, scale, zero)
    M = x.shape[0]
    out = torch.empty((M, N), dtype=torch.float16, device=x.device) if out is None else out
    ws_n = workspace_bytes(OP_GEMM_DECOMP_FUSED, M, K, N, G, 0)
    if workspace is None and ws_n:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=x.device)
    _check("w4_gemm_decomp_fixed_fused", lib().w4_gemm_decomp_fixed_fused(
        _ptr(x), M, K, N, _ptr(packed), _ptr(scale), _ptr(zero), G, _ptr(out), _ptr(tok_scale_out),
        _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(stream)))
    return out if tok_scale_out is None else (out, tok_scale_out)


def stream_read(buf, xor_acc, *, stream=None):
    """A plain read of the device tensor buf (16-byte multiple): XORs its
    32-bit words into xor_acc[0], xor_acc[64], ..., xor_acc[448] (an int32
    device tensor of at least STREAM_READ_ACC_WORDS elements)."""
    if not (buf.is_cuda and buf.is_contiguous()):
        raise ValueError("buf must be a contiguous CUDA tensor")
    _dev(xor_acc, torch.int32, "xor_acc")
    if xor_acc.numel() < STREAM_READ_ACC_WORDS:
        raise ValueError(f"xor_acc needs {STREAM_READ_ACC_WORDS} int32 elements")
    nbytes = buf.numel() * buf.element_size()
    _check("w4_stream_read", lib().w4_stream_read(_ptr(buf), nbytes, _ptr(xor_acc), _stream(stream)))
    return xor_acc


def mfma_rate(kind: int, valu: int, workgroups: int, iters: int, sink, ticks=None, *, stream=None):
    """Independent matrix-core products (kind 0 fp16 16x16x32, 1 int8
    16x16x64), iters x 8 per wave with `valu` fp32 FMAs each; sink: float32
    device tensor of workgroups x 512, ticks: int64 device tensor of
    2 x (workgroups x 8) (shader-clock and 100 MHz ticks per wave) or None."""
    _dev(sink, torch.float32, "sink")
    if sink.numel() < workgroups * 512:
        raise ValueError("sink needs workgroups x 512 elements")
    if ticks is not None:
        _dev(ticks, torch.int64, "ticks")
        if ticks.numel() < workgroups * 16:
            raise ValueError("ticks needs workgroups x 16 elements")
    _check("w4_mfma_rate", lib().w4_mfma_rate(kind, valu, workgroups, iters, _ptr(sink), _ptr(ticks),
                                              _stream(stream)))
    return sink


def salient_select(x, k: int, *, out=None, stream=None):
    """The k salient channels of x [M][K] (int32 indices on x's device)."""
    _dev(x, torch.float16, "x")
    M, K = x.shape
    out = torch.empty((k,), dtype=torch.int32, device=x.device) if out is None else out
    _check("w4_salient_select", lib().w4_salient_select(_ptr(x), M, K, k, _ptr(out), _stream(stream)))
    return out


def residual_correct(x, resid, idx, y, *, stream=None):
    """y += x[:, idx] . resid[idx, :] in place; resid fp16 [K][N], pinned host
    memory (``pin_memory=True``) or a device tensor."""
    _dev(x, torch.float16, "x")
    _dev(y, torch.float16, "y")
    if resid.dtype != torch.float16 or resid.dim() != 2 or not resid.is_contiguous():
        raise ValueError("resid must be a contiguous fp16 [K][N] tensor")
    if resid.device.type == "cpu" and not resid.is_pinned():
        raise ValueError("a host-resident resid must be pinned (pin_memory=True)")
    M, K = x.shape
    N = y.shape[1]
    k = idx.numel()
    _check("w4_residual_correct", lib().w4_residual_correct(_ptr(x), M, K, N, _ptr(resid), _ptr(idx), k, _ptr(y),
                                                            _stream(stream)))
    return y


def residual_correct_f32(x, resid, idx, c=None, *, N=None, stream=None):
    """c = x[:, idx] . resid[idx, :] in fp32 (stored, not added; c fp32
    [M][N], allocated when None); returns c.  With w4.residual_apply(c, y)
    afterwards, y ends as residual_correct would leave it."""
    _dev(x, torch.float16, "x")
    if resid.dtype != torch.float16 or resid.dim() != 2 or not resid.is_contiguous():
        raise ValueError("resid must be a contiguous fp16 [K][N] tensor")
    if resid.device.type == "cpu" and not resid.is_pinned():
        raise ValueError("a host-resident resid must be pinned (pin_memory=True)")
    M, K = x.shape
    N = resid.shape[1] if N is None else N
    c = torch.empty((M, N), dtype=torch.float32, device=x.device) if c is None else c
    _dev(c, torch.float32, "c")
    k = idx.numel()
    _check("w4_residual_correct_f32", lib().w4_residual_correct_f32(_ptr(x), M, K, N, _ptr(resid), _ptr(idx), k,
                                                                    _ptr(c), _stream(stream)))
    return c


def salient_correct_f32(x, resid, k, c=None, *, idx=None, N=None, stream=None):
    """salient_select then residual_correct_f32 in one launch; returns (idx,
    c) with c fp32 [M][N] (allocated when None)."""
    _dev(x, torch.float16, "x")
    if resid.dtype != torch.float16 or resid.dim() != 2 or not resid.is_contiguous():
        raise ValueError("resid must be a contiguous fp16 [K][N] tensor")
    if resid.device.type == "cpu" and not resid.is_pinned():
        raise ValueError("a host-resident resid must be pinned (pin_memory=True)")
    M, K = x.shape
    N = resid.shape[1] if N is None else N
    c = torch.empty((M, N), dtype=torch.float32, device=x.device) if c is None else c
    _dev(c, torch.float32, "c")
    idx = torch.empty((k,), dtype=torch.int32, device=x.device) if idx is None else idx
    _check("w4_salient_correct_f32", lib().w4_salient_correct_f32(_ptr(x), M, K, N, _ptr(resid), k, _ptr(idx),
                                                                  _ptr(c), _stream(stream)))
    return idx, c


def residual_apply(c, y, *, stream=None):
    """y = fp16(y + c) in place (c from residual_correct_f32)."""
    _dev(c, torch.float32, "c")
    _dev(y, torch.float16, "y")
    if c.shape != y.shape or y.dim() != 2:
        raise ValueError("c and y must both be [M][N]")
    M, N = y.shape
    _check("w4_residual_apply", lib().w4_residual_apply(_ptr(c), M, N, _ptr(y), _stream(stream)))
    return y


def salient_correct(x, resid, k, y, *, idx=None, stream=None):
    """salient_select then residual_correct in one launch: y += x[:, idx] .
    resid[idx, :] for the k salient channels; returns idx (int32 [k])."""
    _dev(x, torch.float16, "x")
    _dev(y, torch.float16, "y")
    if resid.dtype != torch.float16 or resid.dim() != 2 or not resid.is_contiguous():
        raise ValueError("resid must be a contiguous fp16 [K][N] tensor")
    if resid.device.type == "cpu" and not resid.is_pinned():
        raise ValueError("a host-resident resid must be pinned (pin_memory=True)")
    M, K = x.shape
    N = y.shape[1]
    idx = torch.empty((k,), dtype=torch.int32, device=x.device) if idx is None else idx
    _check("w4_salient_correct", lib().w4_salient_correct(_ptr(x), M, K, N, _ptr(resid), k, _ptr(idx), _ptr(y),
                                                          _stream(stream)))
    return idx


def quantize_mx(wt, *, codes=None, scale=None, stream=None):
    """MXFP4 of W^T fp32 [N][K]: (codes u8 [N][K], E8M0 scales u8 [N][K/32])."""
    _dev(wt, torch.float32, "wt")
    N, K = wt.shape
    codes = torch.empty((N, K), dtype=torch.uint8, device=wt.device) if codes is None else codes
    scale = torch.empty((N, K // 32), dtype=torch.uint8, device=wt.device) if scale is None else scale
    _check("w4_quantize_mx", lib().w4_quantize_mx(_ptr(wt), K, N, _ptr(codes), _ptr(scale), _stream(stream)))
    return codes, scale


def pack_mx(codes, *, out=None, stream=None):
    """MXFP4 codes [N][K] -> packed tiles (N*K/2 bytes)."""
    _dev(codes, torch.uint8, "codes")
    N, K = codes.shape
    out = torch.empty((N * K // 2,), dtype=torch.uint8, device=codes.device) if out is None else out
    _check("w4_pack_mx", lib().w4_pack_mx(_ptr(codes), K, N, _ptr(out), _stream(stream)))
    return out


def gemm_mx(x, packed, scale, nslices: int = 2, *, out=None, slices_out=None, scales_out=None, workspace=None,
            stream=None):
    """y = x . W' with MXFP4 weights and x split into MXFP4 slices.  Returns y,
    or (y, slices, scales) when an optional output is given."""
    _dev(x, torch.float16, "x")
    _dev(packed, torch.uint8, "packed")
    _dev(scale, torch.uint8, "scale")
    M, K = x.shape
    N = scale.shape[0]
    out = torch.empty((M, N), dtype=torch.float16, device=x.device) if out is None else out
    if workspace is None:
        workspace = torch.empty(workspace_bytes(OP_GEMM_MX, M, K, N, 32, nslices), dtype=torch.uint8,
                                device=x.device)
    _check("w4_gemm_mx", lib().w4_gemm_mx(
        _ptr(x), M, K, N, _ptr(packed), _ptr(scale), nslices, _ptr(out), _ptr(slices_out), _ptr(scales_out),
        _ptr(workspace), workspace.numel(), _stream(stream)))
    if slices_out is None and scales_out is None:
        return out
    return out, slices_out, scales_out


def attn_decode_msd(q, k_packed, k_scale, k_zero, vt_packed, v_scale, v_zero, n_kv: int, *, out=None,
                    workspace=None, stream=None):
    """Decode attention over an INT4 KV cache with MSD on both products.
    q fp16 [B][Hq][128]; caches as documented for w4_attn_decode_msd
    (k_scale [B][Hkv][L] etc.).  Returns out fp16 [B][Hq][128]."""
    _dev(q, torch.float16, "q")
    B, Hq, d = q.shape
    L = k_scale.shape[-1]
    out = torch.empty_like(q) if out is None else out
    if workspace is None:
        workspace = torch.empty(workspace_bytes(OP_ATTN_MSD, B, Hq, L, 0, 0), dtype=torch.uint8, device=q.device)
    _check("w4_attn_decode_msd", lib().w4_attn_decode_msd(
        _ptr(q), B, Hq, n_kv, L, d, _ptr(k_packed), _ptr(k_scale), _ptr(k_zero), _ptr(vt_packed), _ptr(v_scale),
        _ptr(v_zero), _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out

