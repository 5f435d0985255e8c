"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and names shapes; it holds none of the
quantization or matmul arithmetic, so the oracle and the HIP path stay
independent.  All draws use NumPy's PCG64 (``default_rng``) with
``seed = 1000 * cfg + 10 * matrix_idx + role`` (role 0: weight, 1: activations,
2: outlier channel indices).

Distributions follow the workloads of the pages' evaluations, which ran on
trained LLM layers (Gemma 27B, Qwen3 32B, Llama3.3 70B on the
"Fast NF4 Dequantization Kernels" page, Abstract); no checkpoints exist here,
so random layers of those shapes stand in:

* weights W^T [N][K]: fp32, i.i.d. normal with standard deviation 0.02;
* activations x [M][K]: fp32 standard normal rounded to fp16; where the
  workload has outlier channels, ceil(1% of K) distinct K indices (drawn
  without replacement) are multiplied by 20 for every token before rounding.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

WEIGHT_STD = 0.02
OUTLIER_FRACTION = 0.01
OUTLIER_GAIN = 20.0

FMT_INT4_ASYM = 0
FMT_NF4 = 1


def seed_for(cfg: int, matrix_idx: int, role: int) -> int:
    return 1000 * cfg + 10 * matrix_idx + role


def make_weight(cfg: int, matrix_idx: int, N: int, K: int) -> np.ndarray:
    """W^T [N][K] fp32 ~ N(0, 0.02^2)."""
    rng = np.random.default_rng(seed_for(cfg, matrix_idx, 0))
    w = rng.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(WEIGHT_STD)
    return w


def outlier_channels(cfg: int, matrix_idx: int, K: int) -> np.ndarray:
    rng = np.random.default_rng(seed_for(cfg, matrix_idx, 2))
    n = math.ceil(OUTLIER_FRACTION * K)
    return np.sort(rng.choice(K, size=n, replace=False))


def make_activations(cfg: int, matrix_idx: int, M: int, K: int,
                     outliers: bool = True) -> np.ndarray:
    """x [M][K] fp16: N(0,1) (fp32, then rounded), optional x20 channels."""
    rng = np.random.default_rng(seed_for(cfg, matrix_idx, 1))
    x = rng.standard_normal((M, K), dtype=np.float32)
    if outliers and K > 0:
        x[:, outlier_channels(cfg, matrix_idx, K)] *= np.float32(OUTLIER_GAIN)
    return x.astype(np.float16)


@dataclass(frozen=True)
class Matmul:
    """One weight matrix of a workload: W^T is [N][K]."""
    name: str
    K: int
    N: int


@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    Ms: tuple
    mats: tuple
    fmts: tuple  # (fmt, group) pairs
    outliers: bool = True
    paths: tuple = field(default=())


HIDDEN = 8192
INTER = 28672
KV_DIM = 8 * 128  # 8 kv heads x head_dim 128

WORKLOADS = {
    1: Workload(1, "gemv_k1024_n1024", (1,), (Matmul("w", 1024, 1024),),
                ((FMT_INT4_ASYM, 64), (FMT_NF4, 64)), outliers=False),
    2: Workload(2, "decode_gemv_k8192_n8192", (1, 4, 16), (Matmul("w", 8192, 8192),),
                ((FMT_INT4_ASYM, 128), (FMT_NF4, 64))),
    3: Workload(3, "mlp_gemv", (1, 8, 32),
                (Matmul("up_gate", 8192, 28672), Matmul("down", 28672, 8192)),
                ((FMT_INT4_ASYM, 128), (FMT_NF4, 64))),
    4: Workload(4, "prefill_gemm_m2048_k5120_n25600", (2048,),
                (Matmul("w", 5120, 25600),), ((FMT_INT4_ASYM, 128),),
                paths=("dq_f16", "postscale", "msd2")),
    5: Workload(5, "llama70b_layer", (1, 256),
                (Matmul("q", HIDDEN, HIDDEN), Matmul("k", HIDDEN, KV_DIM),
                 Matmul("v", HIDDEN, KV_DIM), Matmul("o", HIDDEN, HIDDEN),
                 Matmul("gate", HIDDEN, INTER), Matmul("up", HIDDEN, INTER),
                 Matmul("down", INTER, HIDDEN)),
                ((FMT_NF4, 64), (FMT_INT4_ASYM, 128))),
}
