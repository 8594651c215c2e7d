"""Tensors whose dtype, shape, strides or device do not match what a call
reads and writes are refused by the binding before anything is launched (the
C functions receive only pointers and sizes, so an output smaller than
[M, N] would otherwise be written past its end); a call with the corrected
argument then runs and matches the oracle."""
import numpy as np
import pytest

import oracle
from block_scaled_precision_quant_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import block_scaled_precision_quant_amd as mx  # noqa: E402
from gpu_util import assert_close_to_oracle, bf16_out_to_f32, to_dev_bf16, to_dev_u8  # noqa: E402


def test_mismatched_tensors_are_refused_before_launch():
    M, N, K = 32, 2880, 512
    print("case binding checks", M, N, K, flush=True)
    a_bits, b_bits = inputs.make_shape(M, N, K, seed=3)
    bq, bs = oracle.quantize(b_bits)
    a = to_dev_bf16(a_bits)
    dbq, dbs = to_dev_u8(bq), to_dev_u8(bs)
    b_packed = mx.pack_b(dbq, dbs)
    sentinel = torch.full((M + 1, N + 8), 5.0, dtype=torch.bfloat16, device=a.device)
    refused = [
        (TypeError, lambda: mx.gemm(a.float(), b_packed, N)),                       # A not bf16
        (ValueError, lambda: mx.gemm(a[:, ::2], b_packed, N)),                      # A strided along K
        (ValueError, lambda: mx.gemm(a, b_packed[::2], N)),                         # B not contiguous
        (ValueError, lambda: mx.gemm(a, b_packed, N, out=sentinel[:M - 1, :N])),    # C too short
        (ValueError, lambda: mx.gemm(a, b_packed, N, out=sentinel[:M, :N - 1])),    # C too narrow
        (ValueError, lambda: mx.gemm(a, b_packed, N, out=sentinel[:M, :2 * N:2])),  # C strided along N
        (TypeError, lambda: mx.gemm(a, b_packed, N, out=sentinel[:M, :N].float())),  # C not bf16
        (ValueError, lambda: mx.gemm(a, b_packed, N,
                                     workspace=torch.zeros((512, 2), dtype=torch.uint8,
                                                           device=a.device)[:, 0])),  # strided workspace
        (ValueError, lambda: mx.gemm_noalloc(a, b_packed, N, out=sentinel[:M, :N - 16])),
        (ValueError, lambda: mx.pack_b(dbq, dbs[:, :-1])),                          # scales too narrow
        (ValueError, lambda: mx.pack_b(dbq[:, ::2], dbs)),                          # codes strided
        (ValueError, lambda: mx.quant_a(a, out_fp4=torch.empty((M - 1, K // 2), dtype=torch.uint8,
                                                               device=a.device))),
        (ValueError, lambda: mx.gemm_prequant(mx.quant_a_packed(a)[::2], M, b_packed, N, K)),
    ]
    for i, (exc, call) in enumerate(refused):
        with pytest.raises(exc):
            call()
        torch.cuda.synchronize()
        assert bool((sentinel == 5.0).all()), "case %d wrote into C" % i
    c = mx.gemm(a, b_packed, N, out=sentinel[:M, :N])
    torch.cuda.synchronize()
    ref = oracle.reference(a_bits, b_bits)
    assert_close_to_oracle(bf16_out_to_f32(c), ref["c32"], "after the refused calls")
    assert bool((sentinel[M:] == 5.0).all()) and bool((sentinel[:, N:] == 5.0).all())
    assert np.isfinite(bf16_out_to_f32(c)).all()


def test_empty_shapes_return_empty_results():
    """M = 0 or N = 0 through every binding call: empty results of the right
    shape, nothing launched, and a surrounding buffer left as it was; a
    normal call on the same stream afterwards still matches the oracle."""
    M, N, K = 16, 256, 512
    print("case empty shapes", M, N, K, flush=True)
    a_bits, b_bits = inputs.make_shape(M, N, K, seed=11)
    bq, bs = oracle.quantize(b_bits)
    a = to_dev_bf16(a_bits)
    b_packed = mx.pack_b(to_dev_u8(bq), to_dev_u8(bs))
    dev = a.device
    a0 = torch.empty((0, K), dtype=torch.bfloat16, device=dev)
    c = mx.gemm(a0, b_packed, N)
    assert tuple(c.shape) == (0, N)
    c = mx.gemm(a, torch.empty(0, dtype=torch.uint8, device=dev), 0)
    assert tuple(c.shape) == (M, 0)
    assert tuple(mx.gemm(a0, b_packed, N, plan=mx.default_plan(M, N, K)).shape) == (0, N)
    sentinel = torch.full((4, N), 3.0, dtype=torch.bfloat16, device=dev)
    mx.gemm_noalloc(a0, b_packed, N, out=sentinel[:0])
    q, s = mx.quant_a(a0)
    assert tuple(q.shape) == (0, K // 2) and tuple(s.shape) == (0, K // 32)
    ap = mx.quant_a_packed(a0)
    assert ap.numel() == 0
    assert tuple(mx.gemm_prequant(ap, 0, b_packed, N, K).shape) == (0, N)
    empty_b = mx.pack_b(torch.empty((0, K // 2), dtype=torch.uint8, device=dev),
                        torch.empty((0, K // 32), dtype=torch.uint8, device=dev))
    assert empty_b.numel() == 0
    assert mx.workspace_bytes(0, N, K) == 0 and mx.workspace_zero_bytes(M, 0, K) == 0
    torch.cuda.synchronize()
    assert bool((sentinel == 3.0).all())
    c = mx.gemm(a, b_packed, N)
    torch.cuda.synchronize()
    ref = oracle.reference(a_bits, b_bits)
    assert_close_to_oracle(bf16_out_to_f32(c), ref["c32"], "after the empty calls")
