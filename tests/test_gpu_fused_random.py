"""Seeded random shapes and fused plans, the A quantization inside the GEMM
read back value by value (the one-hot-B method of test_gpu_fused_quant.py):
rows past M inside a row block, K-groups past K inside a step, several
wavefronts along K, split K with every reduction, and plans whose A stage
takes several load rounds.  Every element of A must come back as exactly the
oracle's dequantized value."""
import functools

import numpy as np
import pytest

from block_scaled_precision_quant_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import block_scaled_precision_quant_amd as mx  # noqa: E402
from test_gpu_fused_quant import read_back  # noqa: E402

N_CASES = 30
KSW = (1, 2, 3, 4, 6, 7, 8, 12, 14, 16)


@functools.lru_cache(maxsize=1)
def cases():
    rng = np.random.default_rng(777)
    out = []
    while len(out) < N_CASES:
        M = int(rng.integers(1, 201))
        K = 32 * int(rng.integers(1, 33))
        KS = -(-K // 128)
        wk = int(rng.choice([1, 2, 3, 4]))
        ksw = [k for k in KSW if KS % (wk * k) == 0]
        if not ksw:
            continue
        k = int(rng.choice(ksw))
        p = mx.Plan(mx.MODE_FUSED, int(rng.choice([1, 2, 4])), int(rng.choice([1, 2])),
                    int(rng.integers(1, 9)), wk, k, KS // (wk * k), int(rng.choice([0, 1, 2])))
        try:
            mx.check_plan(p, M, K, K)
        except mx.Mxfp4Error:
            continue
        out.append((M, K, p))
    return out


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_fused_plan_reads_back_oracle_values(i):
    M, K, plan = cases()[i]
    print("case fused random", i, M, K, plan, flush=True)
    a, _ = inputs.make_shape(M, 16, K, seed=9000 + i)
    n = read_back(a, plan, label="fused random %d %dx%d %s" % (i, M, K, plan))
    assert n == M * K
