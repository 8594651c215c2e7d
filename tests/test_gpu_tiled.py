"""The tiled large-M kernel (plan mode MXFP4_MODE_TILED) against the oracle,
through the C ABI.

Same bar as the other GEMM parity tests: |C_gpu - C_ref| <= 1e-2*|C_ref| + 1e-2
elementwise.  Shapes cover one 256 x 256 tile, ragged M and N edges inside a
tile, K that ends inside a 128-element step, step counts that leave 0 to 3
steps after the kernel's last group of four, grids whose tile count is not
a multiple of the 8 XCD slots (some workgroups have no tile), and sampled
outputs of large shapes; with K split over workgroups (fp32 partials and
the reduce kernel), ranges that end inside a group of four steps or hold a
single step, N not a multiple of 4, and the prequant entry.
"""
import numpy as np
import pytest

import oracle
from block_scaled_precision_quant_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import block_scaled_precision_quant_amd as mx  # noqa: E402
from gpu_util import assert_close_to_oracle, bf16_out_to_f32, to_dev_bf16, to_dev_u8  # noqa: E402
from test_gpu_gemm import reference, run_gemm  # noqa: E402

TILED = mx.Plan(mx.MODE_TILED, 1, 1, 1, 1, 1, 1)      # 256 x 256 tiles
TILED128 = mx.Plan(mx.MODE_TILED, 1, 1, 2, 1, 1, 1)   # waves_n == 2: 256 x 128 tiles
WIDTHS = pytest.mark.parametrize("plan", [TILED, TILED128], ids=["w256", "w128"])


@pytest.mark.parametrize("M,N,K", [
    (256, 256, 128),    # one tile, one K step
    (1, 16, 32),        # one row, one column tile, one K group
    (300, 520, 640),    # ragged M and N; 5 K steps
    (257, 272, 160),    # one row past a tile; K ends inside the second step
    (768, 768, 256),    # 9 tiles: 16 workgroup slots, 7 without a tile
    (513, 1000, 1504),  # N not a multiple of 16, K = 11.75 steps
    (2048, 1040, 2080),
    (300, 280, 384),    # 3 K steps: only the steps after the last group of four
    (520, 512, 800),    # 7 K steps, the last partial: one group of four, then 3
    # the copies' cache policy follows the grid: at most four row tiles
    # stream B nontemporal, at most eight column tiles stream A
    (1300, 1000, 1024),  # 6 row tiles, 4 or 8 column tiles: A nontemporal, B not
    (520, 2200, 512),    # 3 row tiles, 9 or 18 column tiles: B nontemporal, A not
])
@WIDTHS
def test_tiled_full_oracle(M, N, K, plan):
    print("case tiled", M, N, K, plan.waves_n, flush=True)
    ref = reference((M, N, K, M * 7 + N))
    assert_close_to_oracle(run_gemm(ref, plan), ref["c32"], "tiled %dx%dx%d %s" % (M, N, K, plan))


@pytest.mark.parametrize("name", ["m256_n3072_k1536", "m64_n7168_k2048", "m16_n2112_k7168"])
@WIDTHS
def test_tiled_workloads(name, plan):
    print("case tiled", name, plan.waves_n, flush=True)
    ref = reference(name)
    assert_close_to_oracle(run_gemm(ref, plan), ref["c32"], "tiled %s %s" % (name, plan))


def test_tiled_prequant_entry_and_repeat():
    """gemm_prequant with a tiled plan equals the fused-entry tiled call bit
    for bit (same packed A, same kernel), a second call repeats it, and the
    256 x 128 tiles give the same bits as the 256 x 256 ones."""
    M, N, K = 520, 300, 1024
    ref = reference((M, N, K, 11))
    a = to_dev_bf16(ref["a_bits"])
    b_packed = mx.pack_b(to_dev_u8(ref["bq"]), to_dev_u8(ref["bs"]))
    ap = mx.quant_a_packed(a)
    c1 = mx.gemm_prequant(ap, M, b_packed, N, K, plan=TILED)
    c2 = mx.gemm_prequant(ap, M, b_packed, N, K, plan=TILED)
    c3 = mx.gemm(a, b_packed, N, plan=TILED)
    c4 = mx.gemm_prequant(ap, M, b_packed, N, K, plan=TILED128)
    torch.cuda.synchronize()
    assert_close_to_oracle(bf16_out_to_f32(c1), ref["c32"], "tiled gemm_prequant")
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))
    assert torch.equal(c1.view(torch.int16), c3.view(torch.int16))
    # both tile widths run the same products per output in the same order
    assert torch.equal(c1.view(torch.int16), c4.view(torch.int16))


@pytest.mark.parametrize("M,N,K,extra", [
    (260, 200, 384, 37),  # ldc not a multiple of 8: the value-by-value store
    (300, 512, 384, 64),  # whole tiles along N, ldc % 8 == 0: rows staged through LDS
])
@WIDTHS
def test_tiled_strided_output(M, N, K, extra, plan):
    """ldc > N: only the M x N block of C is written."""
    print("case tiled ldc", M, N, K, extra, plan.waves_n, flush=True)
    ref = reference((M, N, K, 5))
    a = to_dev_bf16(ref["a_bits"])
    b_packed = mx.pack_b(to_dev_u8(ref["bq"]), to_dev_u8(ref["bs"]))
    big = torch.full((M + 3, N + extra), 7.0, dtype=torch.bfloat16, device=a.device)
    view = big[:M, :N]
    mx.gemm(a, b_packed, N, out=view, plan=plan)
    torch.cuda.synchronize()
    assert_close_to_oracle(bf16_out_to_f32(view), ref["c32"], "tiled ldc")
    assert bool((big[:, N:] == 7.0).all()) and bool((big[M:, :] == 7.0).all())


@WIDTHS
def test_tiled_max_k_sampled(plan):
    """K at the tiled mode's limit (2^22, 32768 K steps: the largest offsets
    the per-workgroup buffer descriptors carry), ragged M and N.  Elements
    are integers in [-2, 2] (drawn on the GPU from a seeded generator): they
    quantize exactly, every product is an integer of magnitude <= 4 and every
    partial sum an integer of magnitude <= 2^24, so the fp32 sums of the
    oracle and of the kernel are exact in any order and the usual tolerance
    measures the kernel alone.  B is prepared by the packed quantizer
    (bit-exact to the oracle's quantization in test_gpu_quant); the oracle
    quantizes the sampled bf16 rows of A and B itself."""
    M, N, K = 272, 136, 1 << 22
    print("case tiled max K", M, N, K, plan.waves_n, flush=True)
    gen = torch.Generator(device="cuda").manual_seed(4194304)
    a = torch.randint(-2, 3, (M, K), generator=gen, device="cuda", dtype=torch.int8).to(torch.bfloat16)
    b = torch.randint(-2, 3, (N, K), generator=gen, device="cuda", dtype=torch.int8).to(torch.bfloat16)
    b_packed = mx.quant_a_packed(b)
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    mx.gemm(a, b_packed, N, out=c, plan=plan)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 271])
    cols = np.array([0, 15, 127, 128, 135])

    def host_bits(t, idx):
        return t[torch.as_tensor(idx, device=t.device)].view(torch.int16).cpu().numpy().view(np.uint16)

    aq, asc = oracle.quantize(host_bits(a, rows))
    bq, bsc = oracle.quantize(host_bits(b, cols))
    want, want64 = oracle.gemm(oracle.dequantize(aq, asc), oracle.dequantize(bq, bsc))
    assert np.array_equal(want.astype(np.float64), want64)  # the sums are exact
    r = torch.as_tensor(rows, device=c.device)
    q = torch.as_tensor(cols, device=c.device)
    assert_close_to_oracle(bf16_out_to_f32(c[r][:, q]), want, "tiled max K")
    assert not torch.isnan(c).any().item()


@pytest.mark.parametrize("M,N,K", [(1024, 8192, 8192), (4096, 4096, 1024), (8200, 2056, 512),
                                   (272, 512, 65536)])  # 512 K steps: long copies offsets
@WIDTHS
def test_tiled_large_sampled(M, N, K, plan):
    print("case tiled sampled", M, N, K, plan.waves_n, flush=True)
    a, b = inputs.make_shape(M, N, K, seed=(M * 13 + N) % 1000)
    aq, asc = oracle.quantize(a)
    bq, bsc = oracle.quantize(b)
    dev_a = to_dev_bf16(a)
    b_packed = mx.pack_b(to_dev_u8(bq), to_dev_u8(bsc))
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev_a.device)
    mx.gemm(dev_a, b_packed, N, out=c, plan=plan)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M + N + K)
    # the first and last rows and columns of tiles, and random ones
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1, M // 2], rng.integers(0, M, 11)]))
    cols = np.unique(np.concatenate([[0, 255, 256, N - 1, N // 2], rng.integers(0, N, 61)]))
    ad = oracle.dequantize(aq[rows], asc[rows])
    bd = oracle.dequantize(bq[cols], bsc[cols])
    want, _ = oracle.gemm(ad, bd, want64=False)
    r = torch.as_tensor(rows, device=c.device)
    q = torch.as_tensor(cols, device=c.device)
    assert_close_to_oracle(bf16_out_to_f32(c[r][:, q]), want, "tiled %dx%dx%d sampled" % (M, N, K))
    assert not torch.isnan(c).any().item()


@pytest.mark.parametrize("M,N,K,split", [
    (300, 520, 640, 2),     # 5 K steps: ranges of 4 and 1
    (257, 272, 1504, 3),    # K ends inside the 12th step: three ranges of 4
    (513, 1000, 2080, 3),   # 17 steps: 8, 8 and 1; N not a multiple of 16
    (300, 518, 640, 2),     # N % 4 != 0: partials stored value by value
    (768, 768, 4096, 8),    # 32 steps: eight ranges of 4; 9 tiles x 8 workgroups
    (256, 256, 128, 1),
])
@WIDTHS
def test_tiled_split_oracle(M, N, K, split, plan):
    """K shared among split workgroups per tile, fp32 partials summed by the
    reduce kernel: within the GEMM tolerance of the oracle."""
    p = mx.Plan(mx.MODE_TILED, 1, 1, plan.waves_n, 1, 1, split, mx.REDUCE_KERNEL)
    print("case tiled split", M, N, K, split, plan.waves_n, flush=True)
    ref = reference((M, N, K, M * 5 + split))
    assert_close_to_oracle(run_gemm(ref, p), ref["c32"], "tiled split %dx%dx%d %s" % (M, N, K, p))


def test_tiled_split_prequant_and_no_stale_partials():
    """The prequant entry with a split tiled plan equals the fused-entry call
    bit for bit; on one workspace, A then -A gives exactly -C (every partial
    is rewritten by each call)."""
    M, N, K = 520, 300, 3072  # 24 steps: three ranges of 8
    p = mx.Plan(mx.MODE_TILED, 1, 1, 2, 1, 1, 3, mx.REDUCE_KERNEL)
    ref = reference((M, N, K, 17))
    a = to_dev_bf16(ref["a_bits"])
    b_packed = mx.pack_b(to_dev_u8(ref["bq"]), to_dev_u8(ref["bs"]))
    ws = mx.new_workspace(mx.workspace_bytes(M, N, K, p), a.device)
    c1 = mx.gemm(a, b_packed, N, workspace=ws, plan=p)
    c2 = mx.gemm(-a, b_packed, N, workspace=ws, plan=p)
    ap = mx.quant_a_packed(a)
    c3 = mx.gemm_prequant(ap, M, b_packed, N, K, plan=p)
    torch.cuda.synchronize()
    assert_close_to_oracle(bf16_out_to_f32(c1), ref["c32"], "tiled split")
    # values, not bits: an output whose products cancel exactly is +0 for A and for -A
    assert np.array_equal(bf16_out_to_f32(c2), -bf16_out_to_f32(c1))
    assert torch.equal(c1.view(torch.int16), c3.view(torch.int16))


@pytest.mark.parametrize("M,N,K,split", [(256, 8192, 28672, 4), (384, 4104, 16384, 3)])
def test_tiled_split_large_sampled(M, N, K, split):
    p = mx.Plan(mx.MODE_TILED, 1, 1, 2, 1, 1, split, mx.REDUCE_KERNEL)
    print("case tiled split sampled", M, N, K, split, flush=True)
    a, b = inputs.make_shape(M, N, K, seed=(M * 7 + N) % 1000)
    aq, asc = oracle.quantize(a)
    bq, bsc = oracle.quantize(b)
    dev_a = to_dev_bf16(a)
    b_packed = mx.pack_b(to_dev_u8(bq), to_dev_u8(bsc))
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev_a.device)
    mx.gemm(dev_a, b_packed, N, out=c, plan=p)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M + N + K)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1, M // 2], rng.integers(0, M, 11)]))
    cols = np.unique(np.concatenate([[0, 127, 128, N - 1, N // 2], rng.integers(0, N, 61)]))
    rows, cols = rows[rows < M], cols[cols < N]
    want, _ = oracle.gemm(oracle.dequantize(aq[rows], asc[rows]), oracle.dequantize(bq[cols], bsc[cols]),
                          want64=False)
    r = torch.as_tensor(rows, device=c.device)
    q = torch.as_tensor(cols, device=c.device)
    assert_close_to_oracle(bf16_out_to_f32(c[r][:, q]), want, "tiled split %dx%dx%d sampled" % (M, N, K))
    assert not torch.isnan(c).any().item()
