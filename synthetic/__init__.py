"""Seeded synthetic workloads shared by the oracle tests, the GPU parity tests,
the smoke check and the benchmark.

This module only draws random numbers and states shapes.  It holds none of
the method's arithmetic (no thresholds, scales, rounding or matmul), so the
oracle and the HIP path remain independent: both receive the very same
host buffers from here.

The shapes follow the pages' workloads:
  * the ChatGLM2-6B MatMul with L = (max_length x 4096) and R = (4096 x 27392),
    decode with one token and prefill padded to max_length 512
    ("探索ChatGLM2在算能BM1684X上INT8量化部署", sections 3 and 4);
  * a Transformer-big FFN (1024 -> 4096) at 4096 batch tokens, the
    max_batch_tokens of the LightSeq layer config (LightSeq int8 article,
    section 量化训练);
  * the weight distribution: Gaussian with 0.1 % outliers (GOBO review,
    section 提出的方法).
No dataset or trained checkpoint is read: the tensors stand in for them.

Recipe (numpy >= 2, ``rng = np.random.default_rng(seed)``, in this order):
  1. X = rng.standard_normal((M, K), dtype=float32).astype(float16)
  2. W = rng.standard_normal((N, K), dtype=float32) * float32(0.02)
  3. outliers only: idx = rng.choice(N*K, size=round(0.001*N*K), replace=False);
     W.flat[idx] = rng.standard_normal(len(idx), dtype=float32) * float32(0.2)
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    m: int
    k: int
    n: int
    clip_percentile: float = 100.0
    outlier_fraction: float = 0.0
    weight_std: float = 0.02
    outlier_std: float = 0.2
    seed: int = 0

    @property
    def gemm_flops(self) -> int:
        return 2 * self.m * self.n * self.k


# The five workloads.  Order matters: index 0 is the small case the oracle
# finishes in milliseconds, index 1 is the decode GEMV the headline figure is
# quoted on, index 3 the prefill GEMM.
WORKLOADS = (
    Workload("tiny_m1_k256_n512", m=1, k=256, n=512),
    Workload("chatglm2_decode_m1_k4096_n27392", m=1, k=4096, n=27392),
    Workload("small_batch_m8_k4096_n4608", m=8, k=4096, n=4608),
    Workload("chatglm2_prefill_m512_k4096_n27392", m=512, k=4096, n=27392),
    Workload("transformer_big_ffn_outliers_m4096_k1024_n4096", m=4096, k=1024, n=4096,
             clip_percentile=99.99, outlier_fraction=0.001),
)

BY_NAME = {w.name: w for w in WORKLOADS}


def make_inputs(wl: Workload, seed: int | None = None):
    """Return (X float16 [M,K], W float32 [N,K]) for a workload."""
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    x = rng.standard_normal((wl.m, wl.k), dtype=np.float32).astype(np.float16)
    w = rng.standard_normal((wl.n, wl.k), dtype=np.float32)
    w *= np.float32(wl.weight_std)
    if wl.outlier_fraction > 0.0:
        count = int(round(wl.outlier_fraction * wl.n * wl.k))
        idx = rng.choice(wl.n * wl.k, size=count, replace=False)
        vals = rng.standard_normal(count, dtype=np.float32) * np.float32(wl.outlier_std)
        w.reshape(-1)[idx] = vals
    return x, w


def random_x(m: int, k: int, seed: int):
    """Standard-normal fp16 activations of any shape (edge-case tests)."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((m, k), dtype=np.float32).astype(np.float16)


def random_w(n: int, k: int, seed: int, std: float = 0.02):
    """Gaussian fp32 weights of any shape (edge-case tests)."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, k), dtype=np.float32)
    w *= np.float32(std)
    return w
