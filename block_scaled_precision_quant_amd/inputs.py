"""Seeded synthetic inputs for the MXFP4 GEMM workloads.

This module holds the input recipe only -- random draws and the fp32 -> bf16
rounding of those draws -- and none of the quantization or GEMM arithmetic.
Both the HIP path's tests/benchmark and the CPU oracle take their inputs from
here, so the two see identical bits.

Recipe per workload (``numpy.random.default_rng(seed)``, PCG64):
  1. A = standard normal fp32 [M, K];
  2. for the outlier workload, ``n_outliers`` distinct flat positions of A are
     drawn with ``rng.choice(M*K, n_outliers, replace=False)`` and multiplied
     by ``outlier_scale``;
  3. B = ``b_sigma`` * standard normal fp32 [N, K];
  4. both are rounded to bf16 with round-to-nearest-even on the bit pattern.

The shapes are the six benchmark shapes of the amd-mxfp4-mm leaderboard
pages; the value distributions are the synthetic stand-ins described with
each entry (the leaderboard's own generator is not published on the pages).
"""
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    seed: int
    b_sigma: float = 1.0
    n_outliers: int = 0
    outlier_scale: float = 1.0
    note: str = ""


WORKLOADS = {
    w.name: w
    for w in [
        Workload("m4_n2880_k512", 4, 2880, 512, seed=1, note="smallest M; memory floor"),
        Workload("m32_n4096_k512", 32, 4096, 512, seed=2),
        Workload("m32_n2880_k512", 32, 2880, 512, seed=3),
        Workload("m16_n2112_k7168", 16, 2112, 7168, seed=4, n_outliers=1147, outlier_scale=50.0,
                 note="thin grid, long K; 1% of A scaled by 50"),
        Workload("m64_n7168_k2048", 64, 7168, 2048, seed=5, b_sigma=0.02,
                 note="weight-like B, sigma 0.02"),
        Workload("m256_n3072_k1536", 256, 3072, 1536, seed=6, note="compute-leaning"),
    ]
}

# Order used by reports: the six shapes as the pages list them by M.
ORDER = ["m4_n2880_k512", "m32_n4096_k512", "m32_n2880_k512", "m16_n2112_k7168",
         "m64_n7168_k2048", "m256_n3072_k1536"]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the bits as uint16.

    Inputs are finite; NaN handling is not needed for these draws."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 values."""
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make(w, seed=None):
    """Return (A, B) bf16 bit arrays, uint16 [M, K] and [N, K], for a workload.

    ``w`` is a Workload or its name; ``seed`` overrides the workload's seed
    (fresh-seed re-checks use seed + 1000)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(w.seed if seed is None else seed)
    a = rng.standard_normal((w.M, w.K), dtype=np.float32)
    if w.n_outliers:
        idx = rng.choice(w.M * w.K, w.n_outliers, replace=False)
        a.reshape(-1)[idx] *= np.float32(w.outlier_scale)
    b = rng.standard_normal((w.N, w.K), dtype=np.float32) * np.float32(w.b_sigma)
    return f32_to_bf16_bits(a), f32_to_bf16_bits(b)


def make_shape(M, N, K, seed, b_sigma=1.0):
    """Inputs of an arbitrary shape with the default recipe (A and B normal)."""
    return make(Workload("custom", M, N, K, seed=seed, b_sigma=b_sigma))
