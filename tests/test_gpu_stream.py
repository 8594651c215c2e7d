"""Weight-streaming shapes (small M, B of 100-150 MB) through the C ABI,
checked on sampled outputs against the oracle.

The library quantizes B on the GPU and packs it (as a caller would); the
oracle quantizes, from the same bf16 inputs, only the sampled rows of B and
the rows of A, and takes their fp32 dot products.  The plans are the default
one and the split-K plans these sizes run (long K split over workgroups, the
fp32 partials summed by the reduce kernel).  Same bar as every GEMM parity
test: |C_gpu - C_ref| <= 1e-2*|C_ref| + 1e-2 elementwise; C is poisoned with
NaN first and must hold no NaN afterwards.
"""
import numpy as np
import pytest

import oracle
from block_scaled_precision_quant_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import block_scaled_precision_quant_amd as mx  # noqa: E402
from gpu_util import assert_close_to_oracle, bf16_out_to_f32, to_dev_bf16  # noqa: E402

F, P = mx.MODE_FUSED, mx.MODE_PREQUANT

CASES = [
    ((64, 16384, 16384), None),                               # default plan
    ((1, 16384, 16384), mx.Plan(F, 1, 1, 7, 1, 16, 8, 0)),    # fused, 8-way split
    ((16, 8192, 28672), None),                                # default plan, 224 K steps
    ((32, 28672, 8192), mx.Plan(P, 2, 1, 4, 2, 16, 2, 0)),    # pre-quantized A, 2-way split
]


def _id(case):
    (M, N, K), p = case
    return "%dx%dx%d-%s" % (M, N, K, "default" if p is None else
                            "m%d_s%d" % (p.mode, p.split_k))


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_stream_shape_sampled(case):
    (M, N, K), plan = case
    print("case stream", M, N, K, plan or mx.default_plan(M, N, K), flush=True)
    a, b = inputs.make_shape(M, N, K, seed=(M + N + K) % 997)
    dev_a = to_dev_bf16(a)
    dev_b = to_dev_bf16(b)
    bq, bs = mx.quant_a(dev_b)
    del dev_b
    b_packed = mx.pack_b(bq, bs)
    del bq, bs
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev_a.device)
    mx.gemm(dev_a, b_packed, N, out=c, plan=plan)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M * 7 + N)
    cols = np.unique(np.concatenate([[0, N - 1, N // 2, 15, 16], rng.integers(0, N, 59)]))
    aq, asc = oracle.quantize(a)
    bq_h, bs_h = oracle.quantize(b[cols])
    want, _ = oracle.gemm(oracle.dequantize(aq, asc), oracle.dequantize(bq_h, bs_h), want64=False)
    got = bf16_out_to_f32(c[:, torch.as_tensor(cols, device=c.device)])
    assert_close_to_oracle(got, want, "%dx%dx%d sampled" % (M, N, K))
    assert not torch.isnan(c).any().item()
    del c, b_packed, dev_a
    torch.cuda.empty_cache()
