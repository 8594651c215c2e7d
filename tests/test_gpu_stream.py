"""Weight-streaming shapes (small M, B of 100-150 MB) through the C ABI,
checked on sampled outputs against the oracle.

The library quantizes B on the GPU and packs it (as a caller would); the
oracle quantizes, from the same bf16 inputs, only the sampled rows of B and
the rows of A, and takes their fp32 dot products.  The plans are the default
one and the split-K plans these sizes run (long K split over workgroups, the
fp32 partials summed by the reduce kernel); default-plan cases assert the
mode they exercise (the stream kernel with one row block, at M 256..512,
and the tiled kernel with a split of K).  Same bar as every GEMM parity
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
    ((16, 16384, 16384), None),                               # default: stream, one row block
    ((300, 2048, 8192), None),                                # default: stream at M 256..512, ragged M
    ((256, 8192, 28672), None),                               # default: tiled, K split, B nontemporal
]
# the mode each default-plan case is meant to exercise
EXPECT = {(64, 16384, 16384): mx.MODE_STREAM, (16, 8192, 28672): mx.MODE_STREAM,
          (16, 16384, 16384): mx.MODE_STREAM, (300, 2048, 8192): mx.MODE_STREAM,
          (256, 8192, 28672): mx.MODE_TILED}


def _id(case):
    (M, N, K), p = case
    return "%dx%dx%d-%s" % (M, N, K, "default" if p is None else
                            "m%d_s%d" % (p.mode, p.split_k))


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_stream_shape_sampled(case):
    (M, N, K), plan = case
    print("case stream", M, N, K, plan or mx.default_plan(M, N, K), flush=True)
    if plan is None:
        assert mx.default_plan(M, N, K).mode == EXPECT[(M, N, K)]
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


S = mx.MODE_STREAM


def stream_plan(mbw, ntw, steps, M, N, K):
    """A stream-mode plan with `steps` 128-K steps per workgroup."""
    kg = -(-(-(-K // 128)) // 4)
    return mx.Plan(S, mbw, ntw, 4, 1, steps, -(-kg // (steps // 4)), 0)


# shapes the oracle finishes in seconds: ragged M (across row blocks and
# row groups), ragged N, K not a multiple of 128 or of 512, one chunk and
# many, one workgroup along K and several
SMALL = [
    (1, 200, 512, 1, 1, 4),       # one chunk per workgroup, split 1
    (16, 1040, 2080, 1, 2, 8),    # K = 16.25 steps (17 steps, 5 chunks): split 3, last chunk partial
    (37, 264, 4096, 4, 1, 32),    # M across three row blocks, whole K in one workgroup
    (37, 264, 4096, 2, 2, 12),    # two row groups, split 3
    (64, 520, 8192, 4, 2, 64),    # whole K (64 steps) in one workgroup
    (100, 320, 1536, 4, 1, 4),    # two row groups, 12 steps: split 3
    (3, 4096, 640, 1, 2, 8),      # 5 steps: one chunk of four and a partial one
]


@pytest.mark.parametrize("M,N,K,mbw,ntw,steps", SMALL)
def test_stream_mode_against_oracle(M, N, K, mbw, ntw, steps):
    plan = stream_plan(mbw, ntw, steps, M, N, K)
    print("case stream mode", M, N, K, plan, flush=True)
    mx.check_plan(plan, M, N, K)
    a, b = inputs.make_shape(M, N, K, seed=M * 13 + N + K)
    ref = oracle.reference(a, b)
    bq, bs = oracle.quantize(b)
    from gpu_util import to_dev_u8
    b_packed = mx.pack_b(to_dev_u8(bq), to_dev_u8(bs))
    dev_a = to_dev_bf16(a)
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev_a.device)
    mx.gemm(dev_a, b_packed, N, out=c, plan=plan)
    # the same plan on an A quantized beforehand (the prequant entry point)
    c2 = mx.gemm_prequant(mx.quant_a_packed(dev_a), M, b_packed, N, K, plan=plan)
    torch.cuda.synchronize()
    assert_close_to_oracle(bf16_out_to_f32(c), ref["c32"], "stream %dx%dx%d" % (M, N, K))
    assert torch.equal(c.view(torch.int16), c2.view(torch.int16))


@pytest.mark.parametrize("M,N,K,mbw,ntw,steps", [(64, 16384, 16384, 4, 1, 128),
                                                 (16, 8192, 28672, 1, 1, 32),
                                                 (32, 28672, 8192, 2, 2, 64)])
def test_stream_mode_large_sampled(M, N, K, mbw, ntw, steps):
    plan = stream_plan(mbw, ntw, steps, M, N, K)
    print("case stream mode large", M, N, K, plan, flush=True)
    a, b = inputs.make_shape(M, N, K, seed=(M + N + K) % 991)
    dev_a = to_dev_bf16(a)
    dev_b = to_dev_bf16(b)
    bq, bs = mx.quant_a(dev_b)
    del dev_b
    b_packed = mx.pack_b(bq, bs)
    del bq, bs
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev_a.device)
    mx.gemm(dev_a, b_packed, N, out=c, plan=plan)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M * 5 + N)
    cols = np.unique(np.concatenate([[0, N - 1, N // 2, 63, 64], rng.integers(0, N, 59)]))
    aq, asc = oracle.quantize(a)
    bq_h, bs_h = oracle.quantize(b[cols])
    want, _ = oracle.gemm(oracle.dequantize(aq, asc), oracle.dequantize(bq_h, bs_h), want64=False)
    got = bf16_out_to_f32(c[:, torch.as_tensor(cols, device=c.device)])
    assert_close_to_oracle(got, want, "stream mode %dx%dx%d sampled" % (M, N, K))
    assert not torch.isnan(c).any().item()
    del c, b_packed, dev_a
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mbw,ntw,steps", [(4, 2, 1 << 15), (1, 1, 4096)],
                         ids=["whole_k", "split8"])
def test_stream_max_k_sampled(mbw, ntw, steps):
    """K at the stream mode's limit (2^22, 32768 K steps: the largest offsets
    the per-workgroup buffer descriptors carry), ragged M and N, with the
    whole of K in one workgroup (four row blocks, two tiles per wavefront)
    or split eight ways.  Elements are integers in [-2, 2] (drawn on the GPU
    from a seeded generator): they quantize exactly, every product is an
    integer of magnitude <= 4 and every partial sum an integer of magnitude
    <= 2^24, so the fp32 sums of the oracle and of the kernel are exact in
    any order and the usual tolerance measures the kernel alone.  B is
    prepared by the packed quantizer (bit-exact to the oracle's quantization
    in test_gpu_quant); the oracle quantizes the sampled bf16 rows itself."""
    M, N, K = 40, 136, 1 << 22
    plan = stream_plan(mbw, ntw, steps, M, N, K)
    print("case stream max K", M, N, K, plan, flush=True)
    mx.check_plan(plan, M, N, K)
    gen = torch.Generator(device="cuda").manual_seed(4194305)
    a = torch.randint(-2, 3, (M, K), generator=gen, device="cuda", dtype=torch.int8).to(torch.bfloat16)
    b = torch.randint(-2, 3, (N, K), generator=gen, device="cuda", dtype=torch.int8).to(torch.bfloat16)
    b_packed = mx.quant_a_packed(b)
    rows = np.array([0, 1, 15, 16, 39])
    cols = np.array([0, 15, 63, 64, 127, 128, 135])

    def host_bits(t, idx):
        return t[torch.as_tensor(idx, device=t.device)].view(torch.int16).cpu().numpy().view(np.uint16)

    b_rows = host_bits(b, cols)
    del b
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    mx.gemm(a, b_packed, N, out=c, plan=plan)
    torch.cuda.synchronize()
    aq, asc = oracle.quantize(host_bits(a, rows))
    bq, bsc = oracle.quantize(b_rows)
    want, want64 = oracle.gemm(oracle.dequantize(aq, asc), oracle.dequantize(bq, bsc))
    assert np.array_equal(want.astype(np.float64), want64)  # the sums are exact
    r = torch.as_tensor(rows, device=c.device)
    q = torch.as_tensor(cols, device=c.device)
    assert_close_to_oracle(bf16_out_to_f32(c[r][:, q]), want, "stream max K")
    assert not torch.isnan(c).any().item()
    del a, c, b_packed
    torch.cuda.empty_cache()
