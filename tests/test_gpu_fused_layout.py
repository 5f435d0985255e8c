"""GPU parity of products over matrices that share an input stored as one
(q, k and v concatenated along N, as inference engines keep them): the
library's packed bytes, scales and zero points concatenate along N (the tiles
are stored row block by row block), so the concatenated buffers are the
packed form of the concatenated matrix.  Checked against the oracle's product
with the concatenated dequantized weights, for the GEMV, both fp16 GEMM paths
and both MSD products."""
import numpy as np
import pytest
import torch

import bit_weight_quantized_amd as w4
import oracle as o
import workloads as wl
from gpu_helpers import TOL_ROW_REL_L2, announce, dev, host, oracle_weights, require_gpu, row_rel_l2

pytestmark = pytest.mark.gpu

PARTS = ((1024, 512), (1024, 128), (1024, 128))  # q, k, v: (K, N)


CASES = [(fmt, G, path, M) for fmt, G in ((w4.INT4_ASYM, 128), (w4.NF4, 64))
         for path, M in (("gemv", 1), ("gemv", 16), ("dq_f16", 256), ("postscale", 256))]
CASES += [(w4.INT4_ASYM, 128, "msd2", 256), (w4.INT4_ASYM, 128, "msd2_fixed", 256)]  # MSD takes INT4 weights


@pytest.mark.parametrize("fmt,G,path,M", CASES)
def test_concatenated_weights_are_one_matrix(fmt, G, path, M):
    require_gpu()
    K = PARTS[0][0]
    x = wl.make_activations(700 + M, 0, M, K)
    quant, deq = [], []
    for i, (_, N) in enumerate(PARTS):
        w = wl.make_weight(710 + i, 0, N, K)
        codes, scale, zero = oracle_weights(fmt, w, G)
        quant.append((codes, scale, zero))
        deq.append(o.dequant(fmt, codes, scale, zero, G))
    # each part packed and uploaded on its own, then the device buffers joined
    packed = torch.cat([dev(o.pack_w4(c)) for c, _, _ in quant])
    scale = torch.cat([dev(s) for _, s, _ in quant])
    zero = None if fmt == w4.NF4 else torch.cat([dev(z) for _, _, z in quant])
    xd = dev(x)
    announce("fused layout", dict(fmt=fmt, G=G, path=path, M=M))
    if path == "gemv":
        y = w4.gemv(xd, packed, scale, zero, G, fmt)
    elif path in ("dq_f16", "postscale"):
        y = w4.gemm(xd, packed, scale, zero, G, fmt, w4.DQ_F16 if path == "dq_f16" else w4.POSTSCALE)
    elif path == "msd2":
        y = w4.gemm_decomp(xd, packed, scale, zero, G, 2)
    else:
        y = w4.gemm_decomp_fixed(xd, packed, scale, zero, G)
    torch.cuda.synchronize()
    y_ref = o.matmul_ref(x, np.concatenate(deq, axis=0))
    assert row_rel_l2(host(y), y_ref) <= TOL_ROW_REL_L2
    # and each part's columns: the same as that part's own product's, in tolerance
    c0 = 0
    for (c, s, z), (_, N) in zip(quant, PARTS):
        ref_part = o.matmul_ref(x, o.dequant(fmt, c, s, z, G))
        assert row_rel_l2(host(y)[:, c0:c0 + N], ref_part) <= TOL_ROW_REL_L2
        c0 += N
