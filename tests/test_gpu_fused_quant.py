"""The A quantization inside the GEMM, read back value by value.

In fused mode the GEMM quantizes A into LDS and never stores the codes or
scales, so they are observed through the product itself: B is made one-hot
(row n holds a single 1.0 at column k_n, zeros elsewhere).  The oracle
quantizes such a row to scale byte 125 and code 6 in the group of k_n (4 *
2^-2 = 1.0) and to scale byte 0 with zero codes everywhere else, so every
product except one is an exact zero and C[m, n] is exactly the dequantized
value deqA[m, k_n]: at most two significant bits, exact in fp32 and bf16.
Shifting k_n over several calls covers every column of A.

The check is exact equality with the oracle's deqA for every element whose
value is zero or a normal fp32 number (products below 2^-126 may be flushed
by the matrix instruction, and values above the fp32 range overflow; the
linear quantizer's bytes are compared exactly over that whole range in
test_gpu_quant.py).  Equal values for every element of every group leave
only encodings that the product cannot tell apart; the scale rule and the
element rule (submission 752099 `_bf16_to_fp4_hw`, submission 694791
`_mxfp4_quant_tile`) are what make the oracle's values unique.
"""
import numpy as np
import pytest

import oracle
from block_scaled_precision_quant_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import block_scaled_precision_quant_amd as mx  # noqa: E402
from gpu_util import bf16_out_to_f32, to_dev_bf16, to_dev_u8  # noqa: E402
from test_gpu_quant import coverage_matrix  # noqa: E402

F, P, T = mx.MODE_FUSED, mx.MODE_PREQUANT, mx.MODE_TILED
ONE = np.uint16(0x3F80)
FLT_MIN = 2.0 ** -126
FLT_MAX = float(np.finfo(np.float32).max)


def one_hot_b(N, K, shift):
    """B [N, K] with row n one-hot at column (n + shift) % K; returns the
    bits, the column of each row and the oracle's packed B on the device."""
    cols = (np.arange(N) + shift) % K
    b = np.zeros((N, K), dtype=np.uint16)
    b[np.arange(N), cols] = ONE
    bq, bs = oracle.quantize(b)
    # the closed form the test relies on: the group of k_n has scale byte 125
    # and code 6 at k_n, every other group scale byte 0 and zero codes
    want_s = np.zeros((N, K // 32), dtype=np.uint8)
    want_s[np.arange(N), cols // 32] = 125
    want_q = np.zeros((N, K // 2), dtype=np.uint8)
    want_q[np.arange(N), cols // 2] = np.where(cols % 2 == 0, 0x06, 0x60).astype(np.uint8)
    assert np.array_equal(bs, want_s) and np.array_equal(bq, want_q)
    return cols, mx.pack_b(to_dev_u8(bq), to_dev_u8(bs))


def workspace(M, N, K, plan, device):
    nws = mx.workspace_bytes(M, N, K, plan)
    if not nws:
        return None
    ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device=device)
    ws[:mx.workspace_zero_bytes(M, N, K, plan)] = 0
    return ws


def read_back(a_bits, plan, N=None, label=""):
    """Run the GEMM against one-hot B until every column of A has been read
    back, and compare with the oracle's dequantized A.  Returns the number
    of elements compared."""
    M, K = a_bits.shape
    N = N or K
    aq, asc = oracle.quantize(a_bits)
    ad = oracle.dequantize(aq, asc)
    a = to_dev_bf16(a_bits)
    seen = np.zeros((M, K), dtype=bool)
    checked = 0
    for shift in range(0, K, N):
        cols, b_packed = one_hot_b(N, K, shift)
        c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=a.device)
        ws = workspace(M, N, K, plan, a.device)
        mx.gemm(a, b_packed, N, out=c, workspace=ws, plan=plan)
        torch.cuda.synchronize()
        got = bf16_out_to_f32(c).astype(np.float64)
        want = ad[:, cols]
        mag = np.abs(want)
        normal = (mag == 0) | ((mag >= FLT_MIN) & (mag <= FLT_MAX))
        bad = np.argwhere(normal & (got != want))
        if bad.size:
            m, n = bad[0]
            k = cols[n]
            raise AssertionError(
                "%s: %d elements differ; first A[%d, %d] (group %d): gpu %r oracle %r "
                "(oracle scale byte %d, code %d)" % (
                    label, len(bad), m, k, k // 32, got[m, n], want[m, n], asc[m, k // 32],
                    (aq[m, k // 2] >> (4 * (k % 2))) & 0xF))
        checked += int(normal.sum())
        seen[:, cols] = True
    assert seen.all()
    return checked


@pytest.mark.parametrize("name", inputs.ORDER)
def test_default_plan_reads_back_oracle_values(name):
    """Each workload's own shape and default plan (all fused; the thin-grid
    shape splits K seven ways and sums in the reduce kernel), with the
    workload's A, the outlier groups of the thin-grid shape included."""
    w = inputs.WORKLOADS[name]
    plan = mx.default_plan(w.M, w.N, w.K)
    print("case", name, plan, flush=True)
    a, _ = inputs.make(name)
    n = read_back(a, plan, N=w.N, label=name)
    assert n == w.M * w.N * -(-w.K // w.N)  # no element skipped


# Fused plans over the exhaustive coverage groups (every finite bf16
# magnitude under every group maximum at or above it): m_blocks 1, 2 and 4,
# 3, 7 and 12 steps per wavefront, two wavefronts along K, a split K, and a
# wavefront that quantizes many rounds of A before its B loads.
COVERAGE_PLANS = [
    (384, mx.Plan(F, 1, 1, 2, 1, 3, 1)),
    (896, mx.Plan(F, 2, 1, 2, 1, 7, 1)),
    (1536, mx.Plan(F, 4, 1, 2, 1, 12, 1)),
    (1536, mx.Plan(F, 4, 2, 1, 1, 12, 1)),
    (512, mx.Plan(F, 2, 2, 2, 2, 2, 1)),
    (512, mx.Plan(F, 1, 1, 2, 1, 1, 4, mx.REDUCE_KERNEL)),
]


def coverage_rows(K):
    g = coverage_matrix().reshape(-1, 32)
    per_row = K // 32
    rows = -(-g.shape[0] // per_row)
    x = np.zeros((rows * per_row, 32), dtype=np.uint16)
    x[:g.shape[0]] = g
    return x.reshape(rows, K)


@pytest.mark.parametrize("K,plan", COVERAGE_PLANS,
                         ids=lambda x: str(x) if isinstance(x, int) else
                         "mb%d_nt%d_wn%d_wk%d_ks%d_s%d" % (x.m_blocks, x.n_tiles_per_wave, x.waves_n,
                                                          x.waves_k, x.k_steps_per_wave, x.split_k))
def test_coverage_groups_fused(K, plan):
    x = coverage_rows(K)
    print("case coverage", x.shape, plan, flush=True)
    mx.check_plan(plan, x.shape[0], K, K)
    n = read_back(x, plan, label="coverage K=%d %s" % (K, plan))
    assert n > x.size // 2


def special_rows():
    """Ties at unit scale, saturating maxima, all-zero and negative-zero
    groups, negative values that round to zero, all within the fp32 normal
    range after dequantization."""
    groups = []

    def grp(vals):
        v = np.zeros(32, dtype=np.float32)
        v[:len(vals)] = vals
        return v

    groups.append(grp([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25,
                       -1.75, -2.5, -3.5, -5.0]))                      # ties, scale 127
    groups.append(grp([1.625, 0.25, -1.5, 1.0]))                       # saturating max
    groups.append(grp([-1.6875 * 2.0 ** 40, 2.0 ** 38, -(2.0 ** 37)]))  # saturating, large scale
    groups.append(grp([1.7 * 2.0 ** -100, 2.0 ** -102]))               # small scale, normal values
    groups.append(grp([]))                                             # all zero
    groups.append(grp([6.0, -0.2, -0.1, 0.2]))                         # -0.2, -0.1 round to -0
    g = np.stack(groups)
    bits = inputs.f32_to_bf16_bits(g.reshape(-1)).reshape(g.shape)
    neg_zero = np.full((1, 32), 0x8000, dtype=np.uint16)
    return np.concatenate([bits, neg_zero])


@pytest.mark.parametrize("M,K,plan", [
    (37, 544, mx.Plan(F, 2, 1, 1, 5, 1, 1)),                     # 5 waves along K, K ends in a step
    (37, 544, mx.Plan(F, 2, 1, 2, 1, 1, 5, mx.REDUCE_KERNEL)),   # the same K split over workgroups
    (21, 1504, mx.Plan(F, 1, 1, 2, 1, 12, 1)),                   # 47 groups: 11.75 steps
    (70, 800, mx.Plan(F, 4, 1, 1, 1, 7, 1)),                     # rows past M in a 64-row block
    (70, 800, mx.Plan(P, 4, 1, 1, 1, 7, 1)),                     # pre-quantized A
    (300, 1536, mx.Plan(T, 1, 1, 2, 1, 1, 1)),                   # tiled, 256 x 128 tiles
    (300, 1536, mx.Plan(T, 1, 1, 4, 1, 1, 1)),                   # tiled, 256 x 256 tiles
])
def test_ragged_and_special_groups(M, K, plan):
    """Ragged M, K not a multiple of 128, special groups placed in the first
    rows and at the end of K; fused plans, one pre-quantized, two tiled."""
    a, _ = inputs.make_shape(M, 16, K, seed=M * 31 + K)
    sp = special_rows()
    ng = K // 32
    for i in range(sp.shape[0]):
        r, gcol = divmod(i, 2)
        grp_idx = gcol * (ng - 1)  # first and last group of the row
        a[r, 32 * grp_idx:32 * grp_idx + 32] = sp[i]
    print("case ragged", M, K, plan, flush=True)
    mx.check_plan(plan, M, K, K)
    read_back(a, plan, label="%dx%d %s" % (M, K, plan))
