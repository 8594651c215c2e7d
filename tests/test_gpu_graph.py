"""Library calls captured in a HIP graph (torch.cuda.CUDAGraph) replay to the
eager results.

The library allocates nothing and issues only kernel launches on the caller's
stream (no memset nodes: the split-K tile counters and the atomic
accumulator are cleared by the kernels themselves), so a call can be
captured.  Each case runs the call eagerly, captures the same call on the
same buffers, replays the graph several times with eager work and
synchronizations in between, checks every replay against the eager result
(bit for bit; the atomic reduce, whose order of additions is not fixed,
within the GEMM tolerance of the oracle), then writes new values into the
captured input and checks that a replay follows them.  The allocation-free
entry (mxfp4_gemm_noalloc, whose scratch is the library's per-GPU array) is
captured the same way after its first, eager, call.
"""
import numpy as np
import pytest

import oracle
from block_scaled_precision_quant_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import block_scaled_precision_quant_amd as mx  # noqa: E402
from gpu_util import assert_close_to_oracle, bf16_out_to_f32, to_dev_bf16, to_dev_u8  # noqa: E402

F, P, T = mx.MODE_FUSED, mx.MODE_PREQUANT, mx.MODE_TILED

NOALLOC = "noalloc"  # mxfp4_gemm_noalloc: default plan, scratch in the library's array

CASES = [
    ((32, 4096, 512), None),                                           # default: fused
    ((16, 2112, 7168), None),                                          # default: split-K + reduce kernel
    ((16, 2112, 7168), mx.Plan(F, 1, 1, 4, 2, 4, 7, mx.REDUCE_LAST_WG)),
    ((64, 7168, 2048), mx.Plan(F, 4, 1, 2, 1, 4, 4, mx.REDUCE_ATOMIC)),
    ((256, 3072, 1536), mx.Plan(P, 2, 1, 6, 1, 12, 1)),                # quantizer + GEMM
    ((520, 512, 800), mx.Plan(T, 1, 1, 1, 1, 1, 1)),                   # tiled 256 x 256
    ((520, 512, 800), mx.Plan(T, 1, 1, 2, 1, 1, 1)),                   # tiled 256 x 128
    ((520, 512, 1024), mx.Plan(T, 1, 1, 2, 1, 1, 2, mx.REDUCE_KERNEL)),  # tiled, K split in two
    ((32, 8192, 28672), None),                                         # default: stream, split 2 + reduce
    ((40, 520, 4096), mx.Plan(mx.MODE_STREAM, 4, 1, 4, 1, 16, 2, 0)),  # stream, ragged M and N
    ((16, 2112, 7168), NOALLOC),                                       # split-K partials in the array
    ((1024, 4096, 4096), NOALLOC),                                     # pre-quantized A in the array
]


def _id(case):
    (M, N, K), p = case
    return "%dx%dx%d-%s" % (M, N, K, "default" if p is None else p if p == NOALLOC else
                            "m%d_wn%d_s%d_r%d" % (p.mode, p.waves_n, p.split_k, p.split_reduce))


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_graph_replays_match_eager(case):
    (M, N, K), plan = case
    print("case graph", M, N, K, plan, flush=True)
    noalloc = plan == NOALLOC
    if noalloc:
        plan = None
    a_bits, b_bits = inputs.make_shape(M, N, K, seed=M + N + K)
    a2_bits, _ = inputs.make_shape(M, N, K, seed=M + N + K + 1)
    bq, bs = oracle.quantize(b_bits)
    b_packed = mx.pack_b(to_dev_u8(bq), to_dev_u8(bs))
    a = to_dev_bf16(a_bits).contiguous()
    a2 = to_dev_bf16(a2_bits).contiguous()
    atomic = plan is not None and plan.split_k > 1 and plan.split_reduce == mx.REDUCE_ATOMIC
    ws = None if noalloc else mx.new_workspace(mx.workspace_bytes(M, N, K, plan), "cuda")

    def call(src, out):
        if noalloc:  # the eager calls below come first: they look up the array's address
            return mx.gemm_noalloc(src, b_packed, N, out=out)
        return mx.gemm(src, b_packed, N, out=out, workspace=ws, plan=plan)

    eager = call(a, torch.empty((M, N), dtype=torch.bfloat16, device="cuda")).clone()
    eager2 = call(a2, torch.empty((M, N), dtype=torch.bfloat16, device="cuda")).clone()
    torch.cuda.synchronize()

    src = a.clone()
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(src, c)
    torch.cuda.synchronize()

    def check(got, want, label):
        if atomic:
            assert_close_to_oracle(bf16_out_to_f32(got), bf16_out_to_f32(want), label)
        else:
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), label

    scratch = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    for r in range(3):
        c.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        check(c, eager, "replay %d" % r)
        call(a2, scratch)  # eager work on the same workspace between replays
        torch.cuda.synchronize()
        check(scratch, eager2, "eager call between replays %d" % r)
    src.copy_(a2)  # new values in the captured input
    c.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    check(c, eager2, "replay on new input")
    # the eager results themselves against the oracle (shapes it finishes in
    # seconds; the tiled no-alloc case's kernels are checked in test_gpu_tiled.py
    # and its entry against mxfp4_gemm in test_zz_no_alloc.py)
    if M * N * K <= 1.3e9:
        ref = oracle.reference(a_bits, b_bits)
        assert_close_to_oracle(bf16_out_to_f32(eager), ref["c32"], "eager")
