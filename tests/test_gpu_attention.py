"""GPU parity: decode attention over an INT4 KV cache with Multi-Scale Dequant
on both products, against the fp64 oracle of the same computation (and, for
the size of the MSD error, against plain attention over the dequantized
cache)."""
import numpy as np
import pytest
import torch

import bit_weight_quantized_amd as w4
import oracle as o
from gpu_helpers import TOL_ROW_REL_L2, announce, dev, host, require_gpu, row_rel_l2

pytestmark = pytest.mark.gpu
D = 128


def make_cache(seed, B, Hq, Hkv, L, key_outlier=False):
    """Seeded q and caches; the oracle quantizes and packs them."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    k = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    if key_outlier:
        k[0, 0, 5] *= 30.0  # one key far larger: a sharply peaked softmax
    kc = np.zeros((B, Hkv, L, D), np.uint8); vc = np.zeros_like(kc)
    ks = np.zeros((B, Hkv, L), np.float16); kz = np.zeros_like(ks); vs = np.zeros_like(ks); vz = np.zeros_like(ks)
    kp = []; vp = []
    for b in range(B):
        for h in range(Hkv):
            c, s, z = o.quantize_int4_asym(k[b, h], D)
            kc[b, h], ks[b, h], kz[b, h] = c, s[:, 0], z[:, 0]
            kp.append(o.pack_w4(c))
            c, s, z = o.quantize_int4_asym(v[b, h], D)
            vc[b, h], vs[b, h], vz[b, h] = c, s[:, 0], z[:, 0]
            vp.append(o.pack_w4(np.ascontiguousarray(c.T)))  # V^T [d][L]
    return q, (kc, ks, kz), (vc, vs, vz), np.concatenate(kp), np.concatenate(vp)


def run(q, K, V, kp, vp, Hkv):
    return host(w4.attn_decode_msd(dev(q), dev(kp), dev(K[1]), dev(K[2]), dev(vp), dev(V[1]), dev(V[2]), Hkv))


@pytest.mark.parametrize("B,Hq,Hkv,L", [(1, 8, 1, 256), (2, 8, 2, 512), (1, 64, 8, 1024), (2, 16, 1, 768),
                                        (1, 4, 4, 256), (3, 12, 4, 512)])
def test_attention_msd_matches_oracle(B, Hq, Hkv, L):
    require_gpu()
    q, K, V, kp, vp = make_cache(800 + L + Hq, B, Hq, Hkv, L)
    announce("attn msd", dict(B=B, Hq=Hq, Hkv=Hkv, L=L))
    y = run(q, K, V, kp, vp, Hkv)
    for b in range(B):
        ref = o.msd_attention(q[b], K[0][b], K[1][b], K[2][b], V[0][b], V[1][b], V[2][b], Hkv)
        assert row_rel_l2(y[b], ref) <= TOL_ROW_REL_L2


def test_attention_msd_peaked_softmax_and_mean():
    """A single dominant key (the output follows its value) and a zero query
    (uniform weights: the output is the mean of the values)."""
    require_gpu()
    B, Hq, Hkv, L = 1, 8, 1, 512
    q, K, V, kp, vp = make_cache(900, B, Hq, Hkv, L, key_outlier=True)
    q[0, 1] = 0
    announce("attn msd peaked")
    y = run(q, K, V, kp, vp, Hkv)
    ref = o.msd_attention(q[0], K[0][0], K[1][0], K[2][0], V[0][0], V[1][0], V[2][0], Hkv)
    assert row_rel_l2(y[0], ref) <= TOL_ROW_REL_L2
    vd = o.dequant_int4_asym(V[0][0, 0], V[1][0, 0][:, None], V[2][0, 0][:, None], D)
    assert row_rel_l2(y[0, 1:2], vd.mean(axis=0, keepdims=True)) <= TOL_ROW_REL_L2


def test_attention_msd_decode_llama70b_layer():
    """64 query heads over 8 key/value heads, L = 8192 positions: the oracle of
    the same computation, and plain fp64 attention over the dequantized cache
    (the decomposition's own error)."""
    require_gpu()
    B, Hq, Hkv, L = 1, 64, 8, 8192
    q, K, V, kp, vp = make_cache(901, B, Hq, Hkv, L)
    announce("attn msd 64/8 heads, L=8192")
    y = run(q, K, V, kp, vp, Hkv)
    ref = o.msd_attention(q[0], K[0][0], K[1][0], K[2][0], V[0][0], V[1][0], V[2][0], Hkv)
    assert row_rel_l2(y[0], ref) <= TOL_ROW_REL_L2
    kd = np.stack([o.dequant_int4_asym(K[0][0, h], K[1][0, h][:, None], K[2][0, h][:, None], D) for h in range(Hkv)])
    vd = np.stack([o.dequant_int4_asym(V[0][0, h], V[1][0, h][:, None], V[2][0, h][:, None], D) for h in range(Hkv)])
    assert row_rel_l2(y[0], o.attention_ref(q[0], kd, vd, Hkv)) <= TOL_ROW_REL_L2


def test_attention_msd_argument_errors():
    require_gpu()
    B, Hq, Hkv, L = 1, 8, 1, 256
    q, K, V, kp, vp = make_cache(902, B, Hq, Hkv, L)
    with pytest.raises(w4.W4Error) as e:
        w4.attn_decode_msd(dev(q), dev(kp), dev(K[1]), dev(K[2]), dev(vp), dev(V[1]), dev(V[2]), 3)  # 8 % 3
    assert e.value.status == -1


def _call(qd, kd, vd, Hkv, out, ws, stream=None):
    return w4.attn_decode_msd(qd, kd[0], kd[1], kd[2], vd[0], vd[1], vd[2], Hkv, out=out, workspace=ws,
                              stream=stream)


def test_attention_graph_replays_between_eager_calls():
    """Replays of a captured call and eager calls (other queries, same
    workspace, same stream) alternate; every replay's output equals the eager
    output of the same query, and so does every eager call's."""
    require_gpu()
    B, Hq, Hkv, L = 2, 16, 2, 2048
    q, K, V, kp, vp = make_cache(990, B, Hq, Hkv, L)
    q2 = np.random.default_rng(991).standard_normal(q.shape).astype(np.float16)
    qd, q2d = dev(q), dev(q2)
    kd, vd = (dev(kp), dev(K[1]), dev(K[2])), (dev(vp), dev(V[1]), dev(V[2]))
    ws = torch.empty(w4.workspace_bytes(w4.OP_ATTN_MSD, B, Hq, L, 0, 0), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    ref1, ref2, og, o2 = (torch.empty_like(qd) for _ in range(4))
    announce("attn graph replays")
    with torch.cuda.stream(s):
        _call(qd, kd, vd, Hkv, ref1, ws, s)
        _call(q2d, kd, vd, Hkv, ref2, ws, s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _call(qd, kd, vd, Hkv, og, ws, s)
    torch.cuda.synchronize()
    for _ in range(4):
        og.zero_()
        o2.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
            _call(q2d, kd, vd, Hkv, o2, ws, s)
        s.synchronize()
        assert torch.equal(og, ref1)
        assert torch.equal(o2, ref2)
