"""Calls hold no device state of their own: the same calls issued from two
host threads onto two streams, each with its own workspace, give the bits
that the same calls give one after another on one stream.  Plans cover the
fused single launch, split-K with the last-workgroup and atomic reductions
(tile counters and accumulator in the workspace) and the tiled mode.

Both streams are created at the default priority.
"""
import threading

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import block_scaled_precision_quant_amd as mx  # noqa: E402
from block_scaled_precision_quant_amd import inputs  # noqa: E402

SHAPES = [
    (64, 1024, 2048, mx.Plan(mx.MODE_FUSED, 1, 1, 4, 1, 16, 1)),
    (16, 2112, 7168, mx.Plan(mx.MODE_FUSED, 1, 1, 4, 1, 8, 7, mx.REDUCE_LAST_WG)),
    (32, 640, 4096, mx.Plan(mx.MODE_PREQUANT, 1, 1, 2, 1, 8, 4, mx.REDUCE_ATOMIC)),
    (520, 512, 1024, mx.Plan(mx.MODE_TILED, 1, 1, 2, 1, 1, 1)),
]


def _setup(M, N, K, plan, seed):
    a_bits, b_bits = inputs.make_shape(M, N, K, seed=seed)
    to = lambda bits: torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    a = to(a_bits)
    bq, bs = mx.quant_a(to(b_bits))
    return a, mx.pack_b(bq, bs)


def test_two_streams_match_one():
    cases = [(M, N, K, p) + _setup(M, N, K, p, 600 + i) for i, (M, N, K, p) in enumerate(SHAPES)]
    torch.cuda.synchronize()
    # reference: one stream, one call after another
    ref = []
    for M, N, K, p, a, bp in cases:
        ws = mx.new_workspace(mx.workspace_bytes(M, N, K, p), "cuda")
        ref.append(mx.gemm(a, bp, N, workspace=ws, plan=p).clone())
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[None] * len(cases) for _ in streams]
    errors = []

    def worker(k):
        try:
            s = streams[k]
            with torch.cuda.stream(s):
                wss = [mx.new_workspace(mx.workspace_bytes(M, N, K, p), "cuda") for M, N, K, p, _, _ in cases]
                for rep in range(3):
                    for i, (M, N, K, p, a, bp) in enumerate(cases):
                        outs[k][i] = mx.gemm(a, bp, N, workspace=wss[i], plan=p, stream=s)
            s.synchronize()
        except Exception as e:  # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k in range(2):
        for i, (M, N, K, p, _, _) in enumerate(cases):
            got = outs[k][i]
            if p.split_reduce == mx.REDUCE_ATOMIC and p.split_k > 1:
                # atomic adds in varying order: the same values within fp32 rounding
                assert torch.allclose(got.float(), ref[i].float(), rtol=1e-2, atol=1e-2), (k, i)
            else:
                assert torch.equal(got.view(torch.int16), ref[i].view(torch.int16)), (k, i, p)
