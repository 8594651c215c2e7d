"""Seeded random shapes and plans against the oracle, through the C ABI.

Each case draws M in [1, 320], N in [1, 640] and K a multiple of 32 in
[32, 1024], then a plan: the default, the tiled mode, or random plan fields
(fused or pre-quantized A, any row blocks, tiles per wavefront, wavefronts
along N and K, a split of the K steps and a split reduction) kept only when
mxfp4_check_plan accepts them.  Same bar as the other GEMM parity tests:
|C_gpu - C_ref| <= 1e-2*|C_ref| + 1e-2 elementwise, C outside M x N and the
workspace's scratch poisoned with NaN.
"""
import functools

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import block_scaled_precision_quant_amd as mx  # noqa: E402
from gpu_util import assert_close_to_oracle  # noqa: E402
from test_gpu_gemm import reference, run_gemm  # noqa: E402

N_CASES = 40
KSW = (1, 2, 3, 4, 6, 7, 8, 12, 14, 16)


@functools.lru_cache(maxsize=1)
def cases():
    rng = np.random.default_rng(4242)
    out = []
    while len(out) < N_CASES:
        M = int(rng.integers(1, 321))
        N = int(rng.integers(1, 641))
        K = 32 * int(rng.integers(1, 33))
        kind = int(rng.integers(0, 4))
        if kind == 0:
            out.append((M, N, K, None))
            continue
        if kind == 1:
            out.append((M, N, K, mx.Plan(mx.MODE_TILED, 1, 1, 1, 1, 1, 1)))
            continue
        KS = -(-K // 128)
        wk = int(rng.choice([1, 2, 4]))
        ksw = [k for k in KSW if KS % (wk * k) == 0]
        if not ksw:
            continue
        k = int(rng.choice(ksw))
        p = mx.Plan(int(rng.choice([mx.MODE_FUSED, mx.MODE_PREQUANT])), int(rng.choice([1, 2, 4])),
                    int(rng.choice([1, 2])), int(rng.integers(1, 9)), wk, k, KS // (wk * k),
                    int(rng.choice([0, 1, 2])))
        try:
            mx.check_plan(p, M, N, K)
        except mx.Mxfp4Error:
            continue
        out.append((M, N, K, p))
    return out


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_and_plan(i):
    M, N, K, plan = cases()[i]
    print("case random", i, M, N, K, plan, flush=True)
    ref = reference((M, N, K, 5000 + i))
    assert_close_to_oracle(run_gemm(ref, plan), ref["c32"], "random case %d %dx%dx%d %s" % (i, M, N, K, plan))
