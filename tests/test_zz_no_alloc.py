"""mxfp4_gemm_noalloc -- the GEMM with no workspace argument, its scratch in
the library's per-GPU array -- against mxfp4_gemm with a caller workspace,
through the C ABI.  The two run the same default plan and kernels, so their
results must be identical bit for bit.  Each case makes two calls in a row
on the one array, the second with a smaller input, so the second call finds
the first call's partials (or pre-quantized A) still in the array."""
import numpy as np
import pytest

from block_scaled_precision_quant_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import block_scaled_precision_quant_amd as mx  # noqa: E402
from gpu_util import to_dev_bf16  # noqa: E402

# (first shape, second and smaller shape); the default plans of these use the
# scratch for split-K partials (16x2112x7168: 946,176 bytes; 8x2112x7168:
# 473,088), for the pre-quantized A of the tiled kernel (1024x4096x4096:
# 2,228,224) and then of the stream kernel (512x4096x4096: 1,114,112), of
# the pre-quantized plan
# (768x2048x2048: 835,584; 600x3072x2048: 661,504), for the pre-quantized A
# and the split partials of the stream kernel (32x8192x28672: 2,584,576;
# 96x8192x8192: 417,792, no split), or not at all (64x7168x2048, 4x2880x512).
PAIRS = [
    ((16, 2112, 7168), (8, 2112, 7168)),
    ((1024, 4096, 4096), (512, 4096, 4096)),
    ((768, 2048, 2048), (600, 3072, 2048)),
    ((32, 8192, 28672), (96, 8192, 8192)),
    ((64, 7168, 2048), (4, 2880, 512)),
]


def operands(M, N, K, seed):
    a_bits, b_bits = inputs.make_shape(M, N, K, seed=seed)
    a = to_dev_bf16(a_bits)
    bq, bs = mx.quant_a(to_dev_bf16(b_bits))
    return a, mx.pack_b(bq, bs)


@pytest.mark.parametrize("first,second", PAIRS, ids=lambda s: "x".join(map(str, s)))
def test_noalloc_matches_gemm_with_workspace(first, second):
    print("case noalloc", first, second, flush=True)
    for M, N, K in (first, second):
        assert mx.workspace_bytes(M, N, K) <= mx.noalloc_max_scratch_bytes()
    ops = [operands(*s, seed=sum(s)) for s in (first, second)]
    got = []
    for (M, N, K), (a, bp) in zip((first, second), ops):  # back to back, no sync between
        c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=a.device)
        mx.gemm_noalloc(a, bp, N, out=c)
        got.append(c)
    want = []
    for (M, N, K), (a, bp) in zip((first, second), ops):
        ws = mx.new_workspace(mx.workspace_bytes(M, N, K), a.device)
        want.append(mx.gemm(a, bp, N, workspace=ws))
    torch.cuda.synchronize()
    for (M, N, K), g, w in zip((first, second), got, want):
        g, w = g.cpu().view(torch.int16).numpy(), w.cpu().view(torch.int16).numpy()
        assert np.array_equal(g, w), "%dx%dx%d: %d of %d outputs differ" % (
            M, N, K, int((g != w).sum()), g.size)
