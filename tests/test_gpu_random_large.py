"""Seeded random large shapes through the default plan, checked on sampled
outputs against the oracle, through the C ABI.

Each case draws M in [200, 3000], N in [200, 6000] and K a multiple of 32 in
[256, 6144] (M and N need not be multiples of 16, K of 128): the region where
mxfp4_default_plan's cost model chooses between the fused, the pre-quantized
and the tiled modes of either width.  The oracle quantizes all of A and B and
takes the fp32 dot products of sampled rows and columns (the first and last
of each, a tile edge and random ones).  Same bar as the other GEMM parity
tests: |C_gpu - C_ref| <= 1e-2*|C_ref| + 1e-2 elementwise; C is poisoned with
NaN first and must hold no NaN afterwards.
"""
import functools

import numpy as np
import pytest

import oracle
from block_scaled_precision_quant_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import block_scaled_precision_quant_amd as mx  # noqa: E402
from gpu_util import assert_close_to_oracle, bf16_out_to_f32, to_dev_bf16, to_dev_u8  # noqa: E402

N_CASES = 12


@functools.lru_cache(maxsize=1)
def cases():
    rng = np.random.default_rng(777)
    return [(int(rng.integers(200, 3001)), int(rng.integers(200, 6001)), 32 * int(rng.integers(8, 193)))
            for _ in range(N_CASES)]


def _mode(p):
    return {mx.MODE_FUSED: "fused", mx.MODE_PREQUANT: "prequant"}.get(
        p.mode, "tiled%d" % (128 if p.waves_n == 2 else 256))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_large_default_plan(i):
    M, N, K = cases()[i]
    plan = mx.default_plan(M, N, K)
    print("case random large", i, M, N, K, _mode(plan), plan, flush=True)
    a, b = inputs.make_shape(M, N, K, seed=9000 + i)
    aq, asc = oracle.quantize(a)
    bq, bsc = oracle.quantize(b)
    dev_a = to_dev_bf16(a)
    b_packed = mx.pack_b(to_dev_u8(bq), to_dev_u8(bsc))
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev_a.device)
    mx.gemm(dev_a, b_packed, N, out=c)
    torch.cuda.synchronize()
    rng = np.random.default_rng(i)
    rows = np.unique(np.concatenate([[0, M - 1, min(255, M - 1), min(256, M - 1)], rng.integers(0, M, 6)]))
    cols = np.unique(np.concatenate([[0, N - 1, min(127, N - 1), min(128, N - 1)], rng.integers(0, N, 20)]))
    want, _ = oracle.gemm(oracle.dequantize(aq[rows], asc[rows]), oracle.dequantize(bq[cols], bsc[cols]),
                          want64=False)
    r = torch.as_tensor(rows, device=c.device)
    q = torch.as_tensor(cols, device=c.device)
    assert_close_to_oracle(bf16_out_to_f32(c[r][:, q]), want, "random large %dx%dx%d" % (M, N, K))
    assert not torch.isnan(c).any().item()
