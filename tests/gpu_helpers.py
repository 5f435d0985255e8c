"""Helpers for the GPU parity tests: device transfer, oracle-side weight prep,
and the parity metrics.  The oracle side only ever sees seeded inputs and its
own results; nothing computed by the HIP path is fed back into it."""
import sys

import numpy as np
import pytest
import torch

import oracle as o

TOL_ROW_REL_L2 = 2e-3  # max over rows of ||y - y_ref||_2 / ||y_ref||_2


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU: deselect with -m 'not gpu'")


def announce(*parts):
    """Names the case before a GPU step (flushed, so a fault still leaves it)."""
    print("[gpu case]", *parts, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def oracle_weights(fmt, w, G):
    """Oracle quantization of W^T (numpy): codes, scale, zero (None for NF4)."""
    if fmt == o.FMT_INT4_ASYM:
        return o.quantize_int4_asym(w, G)
    codes, absmax = o.quantize_nf4(w, G)
    return codes, absmax, None


def upload_weights(codes, scale, zero):
    """Oracle-packed weights on the device."""
    packed = dev(o.pack_w4(codes))
    return packed, dev(scale), (None if zero is None else dev(zero))


def row_rel_l2(y_gpu, y_ref):
    return o.max_row_rel_l2(np.asarray(y_gpu, dtype=np.float64), y_ref)


def assert_elementwise(y_gpu, y_ref, rel=2.0 ** -10):
    """Per-element guard under the row gate: |y - y_ref| <= rel * (|y_ref| +
    rms of y_ref's row).  A correct kernel's error is the fp16 rounding of
    the output (2^-11 relative) plus fp32 accumulation and, for fp16 weight
    operands, their rounding (about 2^-12 of the row's rms); one wrong zero
    point or scale in a group moves its outputs by a few percent of the
    row's rms, which the row-relative L2 norm over thousands of columns
    would hide."""
    y = np.asarray(y_gpu, dtype=np.float64)
    ref = np.asarray(y_ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    bound = rel * (np.abs(ref) + rms)
    bad = np.abs(y - ref) > bound
    if bad.any():
        m, n = np.argwhere(bad)[0]
        raise AssertionError(f"{int(bad.sum())} outputs beyond the per-element bound; first at [{m},{n}]: "
                             f"{y[m, n]} vs {ref[m, n]} (bound {bound[m, n]:.3g})")
