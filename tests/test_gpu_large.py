"""Large shapes through the C ABI, checked on sampled outputs.

The oracle quantizes all of A and B (cheap), but the fp32 reference dot is
computed only for sampled rows and columns, which it can do one by one.
Shapes exercise long K (a 32-way split), wide grids that keep K inside the
workgroup, and sizes where 32-bit element offsets would overflow.
"""
import numpy as np
import pytest

import oracle
from block_scaled_precision_quant_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import block_scaled_precision_quant_amd as mx  # noqa: E402
from gpu_util import assert_close_to_oracle, bf16_out_to_f32, to_dev_bf16, to_dev_u8  # noqa: E402


@pytest.mark.parametrize("M,N,K", [(1024, 8192, 8192), (4, 16, 131072), (2048, 1040, 2080),
                                   (300, 65536, 256)])
def test_large_shape_sampled(M, N, K):
    print("case", M, N, K, mx.default_plan(M, N, K), flush=True)
    a, b = inputs.make_shape(M, N, K, seed=(M * 31 + N) % 1000)
    aq, asc = oracle.quantize(a)
    bq, bsc = oracle.quantize(b)
    dev_a = to_dev_bf16(a)
    b_packed = mx.pack_b(to_dev_u8(bq), to_dev_u8(bsc))
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev_a.device)
    nws = mx.workspace_bytes(M, N, K)
    ws = mx.new_workspace(nws, dev_a.device) if nws else None
    mx.gemm(dev_a, b_packed, N, out=c, workspace=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M + N + K)
    rows = np.unique(np.concatenate([[0, M - 1, M // 2], rng.integers(0, M, 5)]))
    cols = np.unique(np.concatenate([[0, N - 1, N // 2], rng.integers(0, N, 61)]))
    ad = oracle.dequantize(aq[rows], asc[rows])
    bd = oracle.dequantize(bq[cols], bsc[cols])
    want, _ = oracle.gemm(ad, bd, want64=False)
    got = bf16_out_to_f32(c[torch.as_tensor(rows, device=c.device)][:, torch.as_tensor(cols, device=c.device)])
    assert_close_to_oracle(got, want, "%dx%dx%d sampled" % (M, N, K))
    # every output was written (NaN poison gone)
    assert not torch.isnan(c).any().item()
