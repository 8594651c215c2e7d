"""GPU GEMM parity against the CPU oracle, through the C ABI.

Bar: |C_gpu - C_ref| <= 1e-2*|C_ref| + 1e-2 elementwise, C_ref the oracle's
fp32 sum over the oracle's own quantization of A and B.  B goes to the GPU
as the oracle's fp4/e8m0 bytes and is repacked by mxfp4_pack_b.
"""
import numpy as np
import pytest

import oracle
from block_scaled_precision_quant_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import block_scaled_precision_quant_amd as mx  # noqa: E402
from gpu_util import assert_close_to_oracle, bf16_out_to_f32, to_dev_bf16, to_dev_u8  # noqa: E402

F, P = mx.MODE_FUSED, mx.MODE_PREQUANT

_REF_CACHE = {}


def reference(name_or_shape, seed=None):
    key = (name_or_shape, seed)
    if key not in _REF_CACHE:
        if isinstance(name_or_shape, str):
            a, b = inputs.make(name_or_shape, seed=seed)
        else:
            M, N, K, sd = name_or_shape
            a, b = inputs.make_shape(M, N, K, seed=sd)
        ref = oracle.reference(a, b)
        ref["a_bits"] = a
        _REF_CACHE[key] = ref
        if len(_REF_CACHE) > 4:
            _REF_CACHE.pop(next(iter(_REF_CACHE)))
    return _REF_CACHE[key]


def run_gemm(ref, plan=None, poison=True):
    a = to_dev_bf16(ref["a_bits"])
    M, K = ref["a_bits"].shape
    N = ref["bq"].shape[0]
    b_packed = mx.pack_b(to_dev_u8(ref["bq"]), to_dev_u8(ref["bs"]))
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=a.device)
    ws = workspace(M, N, K, plan, a.device)
    mx.gemm(a, b_packed, N, out=c, workspace=ws, plan=plan)
    torch.cuda.synchronize()
    return bf16_out_to_f32(c)


def workspace(M, N, K, plan, device):
    """Workspace with zeroed tile counters and NaN-poisoned scratch."""
    nws = mx.workspace_bytes(M, N, K, plan)
    if not nws:
        return None
    ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device=device)
    ws[:mx.workspace_zero_bytes(M, N, K, plan)] = 0
    return ws


@pytest.mark.parametrize("name", inputs.ORDER)
def test_workload_default_plan(name):
    print("case", name, mx.default_plan(*[inputs.WORKLOADS[name].__dict__[k] for k in "MNK"]),
          flush=True)
    ref = reference(name)
    assert_close_to_oracle(run_gemm(ref), ref["c32"], name)


@pytest.mark.parametrize("name", ["m4_n2880_k512", "m16_n2112_k7168"])
def test_workload_fresh_seed(name):
    seed = inputs.WORKLOADS[name].seed + 1000
    ref = reference(name, seed=seed)
    assert_close_to_oracle(run_gemm(ref), ref["c32"], name + " fresh seed")


PLANS = {
    "m4_n2880_k512": [mx.Plan(F, 1, 1, 1, 1, 4, 1), mx.Plan(F, 1, 1, 4, 1, 4, 1),
                      mx.Plan(F, 1, 1, 1, 4, 1, 1), mx.Plan(F, 1, 2, 2, 2, 2, 1),
                      mx.Plan(P, 1, 1, 2, 1, 4, 1), mx.Plan(F, 1, 1, 2, 1, 2, 2),
                      mx.Plan(P, 1, 2, 1, 1, 1, 4)],
    "m32_n2880_k512": [mx.Plan(F, 2, 1, 2, 1, 4, 1), mx.Plan(F, 2, 2, 4, 1, 4, 1),
                       mx.Plan(F, 1, 1, 2, 2, 2, 1), mx.Plan(P, 2, 1, 4, 1, 4, 1),
                       mx.Plan(P, 1, 1, 2, 1, 2, 2)],
    "m16_n2112_k7168": [mx.Plan(P, 1, 1, 1, 2, 7, 4), mx.Plan(F, 1, 1, 1, 2, 7, 4),
                        mx.Plan(F, 1, 1, 2, 1, 14, 4), mx.Plan(P, 1, 1, 1, 1, 8, 7),
                        mx.Plan(P, 1, 2, 2, 2, 14, 2), mx.Plan(P, 1, 1, 1, 4, 14, 1),
                        mx.Plan(P, 1, 1, 1, 8, 7, 1)],
    "m64_n7168_k2048": [mx.Plan(P, 4, 1, 2, 1, 16, 1), mx.Plan(F, 4, 1, 2, 1, 4, 4),
                        mx.Plan(P, 2, 2, 2, 2, 8, 1), mx.Plan(P, 4, 1, 4, 1, 8, 2),
                        mx.Plan(F, 2, 1, 4, 1, 8, 2)],
    "m256_n3072_k1536": [mx.Plan(P, 4, 1, 4, 1, 12, 1), mx.Plan(P, 4, 2, 2, 1, 12, 1),
                         mx.Plan(P, 2, 1, 4, 2, 6, 1), mx.Plan(P, 4, 1, 2, 1, 3, 4),
                         mx.Plan(F, 4, 1, 2, 1, 6, 2)],
}


@pytest.mark.parametrize("name,plan", [(n, p) for n, ps in PLANS.items() for p in ps],
                         ids=lambda x: str(x) if isinstance(x, str) else
                         "m%d_mb%d_nt%d_wn%d_wk%d_ks%d_s%d" % (x.mode, x.m_blocks,
                                                             x.n_tiles_per_wave, x.waves_n,
                                                             x.waves_k, x.k_steps_per_wave,
                                                             x.split_k))
def test_workload_plan_override(name, plan):
    w = inputs.WORKLOADS[name]
    print("case", name, plan, flush=True)
    mx.check_plan(plan, w.M, w.N, w.K)
    ref = reference(name)
    assert_close_to_oracle(run_gemm(ref, plan), ref["c32"], "%s %s" % (name, plan))


@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (5, 48, 256), (17, 80, 384), (33, 144, 640),
                                   (100, 1008, 1152), (63, 272, 896), (2, 16, 7168),
                                   # general shapes: N not a multiple of 16, K of 32
                                   (1, 1, 32), (5, 24, 96), (3, 40, 160), (17, 100, 544),
                                   (70, 100, 544), (33, 1000, 1504), (9, 17, 4128)])
def test_ragged_shapes_default_plan(M, N, K):
    print("case", M, N, K, mx.default_plan(M, N, K), flush=True)
    ref = reference((M, N, K, M * 7 + N))
    assert_close_to_oracle(run_gemm(ref), ref["c32"], "%dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K,plan", [
    (7, 80, 512, mx.Plan(F, 1, 2, 2, 1, 4, 1)),   # ragged N group (5 tiles over 4)
    (40, 48, 384, mx.Plan(F, 2, 1, 2, 1, 3, 1)),  # ragged M block, KSW=3 scale span
    (40, 48, 768, mx.Plan(P, 4, 1, 1, 1, 6, 1)),
    (20, 64, 1792, mx.Plan(F, 2, 1, 1, 2, 7, 1)),
    (20, 64, 1792, mx.Plan(P, 1, 1, 4, 1, 14, 1)),
])
def test_ragged_shapes_plans(M, N, K, plan):
    print("case", M, N, K, plan, flush=True)
    ref = reference((M, N, K, 99 + M))
    assert_close_to_oracle(run_gemm(ref, plan), ref["c32"], "%dx%dx%d %s" % (M, N, K, plan))


# the pages' correctness shapes (submission 752099's configuration table)
@pytest.mark.parametrize("M,N,K", [(8, 2112, 7168), (16, 3072, 1536), (64, 3072, 1536),
                                   (256, 2880, 512)])
def test_page_test_shapes(M, N, K):
    print("case", M, N, K, mx.default_plan(M, N, K), flush=True)
    ref = reference((M, N, K, M + N + K))
    assert_close_to_oracle(run_gemm(ref), ref["c32"], "%dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K,plan", [
    (17, 100, 544, mx.Plan(F, 1, 1, 2, 1, 1, 5, 0)),
    (17, 100, 544, mx.Plan(P, 2, 2, 1, 1, 1, 5, 1)),
    (5, 24, 96, mx.Plan(F, 1, 2, 1, 1, 1, 1)),
    (33, 1000, 1504, mx.Plan(F, 2, 1, 2, 3, 4, 1)),
    (33, 1000, 1504, mx.Plan(P, 1, 2, 2, 1, 3, 4, 1)),
])
def test_general_shapes_plans(M, N, K, plan):
    print("case", M, N, K, plan, flush=True)
    ref = reference((M, N, K, 7 + M))
    assert_close_to_oracle(run_gemm(ref, plan), ref["c32"], "%dx%dx%d %s" % (M, N, K, plan))


def test_lane_map_one_hot():
    """One-hot A rows against structured B pin rows, columns and K groups."""
    M, N, K = 16, 32, 256
    a = np.zeros((M, K), dtype=np.uint16)
    one = np.uint16(0x3F80)
    ks = [(m * 37 + 5) % K for m in range(M)]
    for m in range(M):
        a[m, ks[m]] = one
    _, b = inputs.make_shape(M, N, K, seed=3)
    ref = oracle.reference(a, b)
    ref["a_bits"] = a
    got = run_gemm(ref, mx.Plan(F, 1, 1, 2, 1, 2, 1))
    for m in range(M):
        np.testing.assert_array_equal(got[m], inputs.bf16_bits_to_f32(
            inputs.f32_to_bf16_bits(ref["bd"][:, ks[m]].astype(np.float32))))


@pytest.mark.parametrize("name,plan", [
    ("m16_n2112_k7168", mx.Plan(F, 1, 1, 4, 2, 4, 7)),
    ("m16_n2112_k7168", mx.Plan(P, 1, 1, 1, 2, 7, 4)),
    ("m64_n7168_k2048", mx.Plan(F, 4, 1, 2, 1, 4, 4)),
    ("m4_n2880_k512", mx.Plan(F, 1, 2, 1, 1, 1, 4)),
])
def test_split_reduce_modes_agree(name, plan):
    """Last-workgroup reduce and the reduce kernel give the same bits, and a
    reused workspace (counters back at zero) gives them again."""
    w = inputs.WORKLOADS[name]
    print("case", name, plan, flush=True)
    ref = reference(name)
    a = to_dev_bf16(ref["a_bits"])
    b_packed = mx.pack_b(to_dev_u8(ref["bq"]), to_dev_u8(ref["bs"]))
    outs = []
    for reduce in (mx.REDUCE_KERNEL, mx.REDUCE_LAST_WG):
        p = mx.Plan(*(list(plan.__dict__.values())[:7] + [reduce]))
        ws = workspace(w.M, w.N, w.K, p, a.device)
        for _ in range(3):
            c = torch.full((w.M, w.N), float("nan"), dtype=torch.bfloat16, device=a.device)
            mx.gemm(a, b_packed, w.N, out=c, workspace=ws, plan=p)
            torch.cuda.synchronize()
            outs.append(bf16_out_to_f32(c))
        nz = mx.workspace_zero_bytes(w.M, w.N, w.K, p)
        assert int(ws[:nz].count_nonzero()) == 0  # counters returned to zero
    assert_close_to_oracle(outs[0], ref["c32"], "%s %s" % (name, plan))
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))


@pytest.mark.parametrize("name,plan", [
    ("m16_n2112_k7168", mx.Plan(F, 1, 1, 4, 2, 4, 7, mx.REDUCE_LAST_WG)),
    ("m16_n2112_k7168", mx.Plan(F, 1, 1, 4, 2, 4, 7, mx.REDUCE_KERNEL)),
    ("m64_n7168_k2048", mx.Plan(F, 4, 1, 2, 1, 4, 4, mx.REDUCE_LAST_WG)),
    ("m4_n2880_k512", mx.Plan(F, 1, 2, 1, 1, 1, 4, mx.REDUCE_LAST_WG)),
])
def test_split_no_stale_partials(name, plan):
    """Back-to-back calls on one workspace with A, then -A: the second call
    must give exactly -C (quantization is sign-symmetric and the K order is
    fixed), so partials left by the first call can never be read back."""
    w = inputs.WORKLOADS[name]
    print("case", name, plan, flush=True)
    ref = reference(name)
    a = to_dev_bf16(ref["a_bits"])
    neg = to_dev_bf16(ref["a_bits"] ^ np.uint16(0x8000))
    b_packed = mx.pack_b(to_dev_u8(ref["bq"]), to_dev_u8(ref["bs"]))
    ws = workspace(w.M, w.N, w.K, plan, a.device)
    outs = []
    for x in (a, neg, a, neg):
        c = torch.full((w.M, w.N), float("nan"), dtype=torch.bfloat16, device=a.device)
        mx.gemm(x, b_packed, w.N, out=c, workspace=ws, plan=plan)
        outs.append(c)  # no synchronization between the calls
    torch.cuda.synchronize()
    outs = [bf16_out_to_f32(c) for c in outs]
    assert_close_to_oracle(outs[0], ref["c32"], "%s %s" % (name, plan))
    for i in range(1, 4):
        want = outs[0] if i % 2 == 0 else -outs[0]
        assert np.array_equal(outs[i], want), (name, plan, i)


@pytest.mark.parametrize("shape,plan", [
    ("m16_n2112_k7168", mx.Plan(F, 1, 1, 4, 2, 4, 7, mx.REDUCE_ATOMIC)),
    ("m16_n2112_k7168", mx.Plan(P, 1, 1, 1, 2, 7, 4, mx.REDUCE_ATOMIC)),
    ("m64_n7168_k2048", mx.Plan(F, 4, 1, 2, 1, 4, 4, mx.REDUCE_ATOMIC)),
    ("m4_n2880_k512", mx.Plan(F, 1, 2, 1, 1, 1, 4, mx.REDUCE_ATOMIC)),
    ((33, 1000, 1504, 40), mx.Plan(F, 1, 2, 2, 1, 3, 4, mx.REDUCE_ATOMIC)),
    ((17, 24, 4128, 41), mx.Plan(F, 2, 1, 1, 3, 1, 11, mx.REDUCE_ATOMIC)),
])
def test_split_atomic_reduce(shape, plan):
    """fp32 atomic adds into one accumulator: within tolerance on every call,
    the accumulator and counters back at zero after each call, and a call on
    -A right after one on A gives -C within tolerance (its order of
    additions differs, so not bit for bit)."""
    print("case", shape, plan, flush=True)
    ref = reference(shape)
    M, K = ref["a_bits"].shape
    N = ref["bq"].shape[0]
    a = to_dev_bf16(ref["a_bits"])
    neg = to_dev_bf16(ref["a_bits"] ^ np.uint16(0x8000))
    b_packed = mx.pack_b(to_dev_u8(ref["bq"]), to_dev_u8(ref["bs"]))
    ws = workspace(M, N, K, plan, a.device)
    nz = mx.workspace_zero_bytes(M, N, K, plan)
    assert nz > M * N * 4
    for i, x in enumerate((a, neg, a)):
        c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=a.device)
        mx.gemm(x, b_packed, N, out=c, workspace=ws, plan=plan)
        torch.cuda.synchronize()
        want = ref["c32"] if i % 2 == 0 else -ref["c32"]
        assert_close_to_oracle(bf16_out_to_f32(c), want, "%s %s call %d" % (shape, plan, i))
        assert int(ws[:nz].count_nonzero()) == 0  # counters and accumulator cleared


def test_bitwise_repeatable():
    ref = reference("m16_n2112_k7168")
    p = mx.default_plan(16, 2112, 7168)
    c1 = run_gemm(ref, p)
    c2 = run_gemm(ref, p)
    assert np.array_equal(c1.view(np.uint32), c2.view(np.uint32))


def test_gemm_prequant_entry():
    """quant_a_packed + gemm_prequant equals the fused call."""
    name = "m64_n7168_k2048"
    ref = reference(name)
    a = to_dev_bf16(ref["a_bits"])
    M, K = ref["a_bits"].shape
    N = ref["bq"].shape[0]
    b_packed = mx.pack_b(to_dev_u8(ref["bq"]), to_dev_u8(ref["bs"]))
    ap = mx.quant_a_packed(a)
    c = mx.gemm_prequant(ap, M, b_packed, N, K)
    torch.cuda.synchronize()
    assert_close_to_oracle(bf16_out_to_f32(c), ref["c32"], "gemm_prequant")


def test_library_quantized_b_matches_oracle_path():
    """B quantized on the GPU by the library (the benchmark's route) gives the
    same packed bytes as the oracle's B."""
    _, b = inputs.make("m4_n2880_k512")
    rq, rs = oracle.quantize(b)
    bq, bs = mx.quant_a(to_dev_bf16(b))
    p1 = mx.pack_b(bq, bs)
    p2 = mx.pack_b(to_dev_u8(rq), to_dev_u8(rs))
    torch.cuda.synchronize()
    assert torch.equal(p1, p2)
