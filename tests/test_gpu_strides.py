"""Strided operands through the GEMM entry points: A a column slice of a
wider bf16 matrix (lda > K) and C a column slice of a wider output
(ldc > N).  Only the M x N block of C may be written: the rest of the wider
buffer is NaN before the call and must stay NaN.  Covers the fused kernel's
A addressing, the reduce kernel's vector and element stores (row starts 8-byte
aligned or not), the in-launch reductions' stores, pre-quantized A and the
allocation-free entry.  Bar: the GEMM tolerance against the oracle."""
import numpy as np
import pytest

import oracle
from block_scaled_precision_quant_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import block_scaled_precision_quant_amd as mx  # noqa: E402
from gpu_util import assert_close_to_oracle, bf16_out_to_f32, to_dev_bf16, to_dev_u8  # noqa: E402

F, P = mx.MODE_FUSED, mx.MODE_PREQUANT
NOALLOC = "noalloc"

CASES = [
    # (M, N, K, lda, ldc, plan)
    (32, 2880, 512, 520, 2900, None),                                      # fused default
    (16, 2112, 7168, 7200, 2120, None),                                    # split 7, reduce kernel, 8-byte rows
    (16, 2112, 7168, 7176, 2113, None),                                    # reduce kernel, unaligned rows
    (16, 2112, 7168, 7176, 2117, mx.Plan(F, 1, 1, 4, 2, 4, 7, mx.REDUCE_LAST_WG)),
    (64, 7168, 2048, 2056, 7171, mx.Plan(F, 4, 1, 2, 1, 4, 4, mx.REDUCE_ATOMIC)),
    (37, 1000, 1504, 1512, 1003, mx.Plan(F, 2, 1, 2, 3, 4, 1)),           # ragged M, N, K
    (256, 3072, 1536, 1544, 3080, mx.Plan(P, 2, 1, 6, 1, 12, 1)),         # pre-quantized A
    (40, 520, 4096, 4104, 523, mx.Plan(mx.MODE_STREAM, 4, 1, 4, 1, 16, 2, 0)),  # stream, split 2
    (16, 2112, 7168, 7200, 2115, NOALLOC),                                 # allocation-free entry
]


@pytest.mark.parametrize("M,N,K,lda,ldc,plan", CASES,
                         ids=lambda x: str(x) if not isinstance(x, mx.Plan) else
                         "m%d_s%d_r%d" % (x.mode, x.split_k, x.split_reduce))
def test_strided_a_and_c(M, N, K, lda, ldc, plan):
    print("case strides", M, N, K, lda, ldc, plan, flush=True)
    a_bits, b_bits = inputs.make_shape(M, N, K, seed=M + N + lda)
    ref = oracle.reference(a_bits, b_bits)
    wide_a = np.zeros((M, lda), dtype=np.uint16)
    wide_a[:, :K] = a_bits
    wide_a[:, K:] = 0x7FC0  # NaN bf16 past K: never read
    a = to_dev_bf16(wide_a)[:, :K]
    assert a.stride(0) == lda
    b_packed = mx.pack_b(to_dev_u8(ref["bq"]), to_dev_u8(ref["bs"]))
    wide_c = torch.full((M, ldc), float("nan"), dtype=torch.bfloat16, device=a.device)
    c = wide_c[:, :N]
    if plan == NOALLOC:
        mx.gemm_noalloc(a, b_packed, N, out=c)
    else:
        nws = mx.workspace_bytes(M, N, K, plan)
        ws = None
        if nws:
            ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device=a.device)
            ws[:mx.workspace_zero_bytes(M, N, K, plan)] = 0
        mx.gemm(a, b_packed, N, out=c, workspace=ws, plan=plan)
    torch.cuda.synchronize()
    got = bf16_out_to_f32(wide_c)
    assert_close_to_oracle(got[:, :N], ref["c32"], "strided %dx%dx%d" % (M, N, K))
    assert np.isnan(got[:, N:]).all(), "C written outside the M x N block"
