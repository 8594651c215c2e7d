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


def _tile_bytes(packed, t, RT, KS, KG):
    """Data and scale bytes of row tile t in an MX-packed buffer of RT tiles."""
    D = RT * KS * 1024
    data = packed[t * KS * 1024:(t + 1) * KS * 1024]
    sc = packed[D + t * KG * 256:D + (t + 1) * KG * 256]
    return torch.cat([data, sc]).cpu().numpy()


def test_quantizers_past_one_item_per_thread():
    """The quantizer grids stop at 2^20 workgroups of 256 threads; past 2^28
    8-element items each thread takes several (grid-stride).  2.2e9 elements,
    drawn on the device from a seeded generator; sampled rows and 16-row
    tiles checked against the oracle and the packed layout's closed form."""
    from gpu_util import pack_host, packed_dims
    M, K = 66000, 32768
    assert M * K // 8 > (1 << 28)
    print("case quant", M, K, flush=True)
    gen = torch.Generator(device="cuda:0").manual_seed(11)
    a = torch.randn((M, K), dtype=torch.bfloat16, device="cuda:0", generator=gen)
    rng = np.random.default_rng(11)
    rows = sorted(set([0, 1, M // 2, M - 2, M - 1] + list(rng.integers(0, M, 5))))
    bits = {r: a[r].view(torch.int16).cpu().numpy().view(np.uint16)[None] for r in rows}
    q, s = mx.quant_a(a)
    torch.cuda.synchronize()
    for r in rows:
        rq, rs = oracle.quantize(bits[r])
        assert np.array_equal(q[r].cpu().numpy(), rq[0]), ("codes", r)
        assert np.array_equal(s[r].cpu().numpy(), rs[0]), ("scales", r)
    del q, s
    packed = mx.quant_a_packed(a)
    torch.cuda.synchronize()
    RT, KS, KG = packed_dims(M, K)
    for t in sorted(set([0, 1, RT // 2, RT - 1] + list(rng.integers(0, RT, 3)))):
        r0, r1 = 16 * t, min(16 * t + 16, M)
        tb = a[r0:r1].view(torch.int16).cpu().numpy().view(np.uint16)
        rq, rs = oracle.quantize(tb)
        assert np.array_equal(_tile_bytes(packed, t, RT, KS, KG), pack_host(rq, rs)), ("tile", t)
    del packed, a
    torch.cuda.empty_cache()


def test_pack_b_past_one_item_per_thread():
    """pack_b past 2^28 work items (N*K = 2^33): random code and scale bytes
    on the device, sampled 16-row tiles against the closed form."""
    from gpu_util import pack_host, packed_dims
    N, K = 1 << 18, 1 << 15
    print("case pack_b", N, K, flush=True)
    gen = torch.Generator(device="cuda:0").manual_seed(12)
    fp4 = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device="cuda:0", generator=gen)
    sc = torch.randint(0, 256, (N, K // 32), dtype=torch.uint8, device="cuda:0", generator=gen)
    packed = mx.pack_b(fp4, sc)
    torch.cuda.synchronize()
    RT, KS, KG = packed_dims(N, K)
    assert RT * KS * 64 + RT * KG * 64 > (1 << 28)
    rng = np.random.default_rng(12)
    for t in sorted(set([0, RT // 2, RT - 1] + list(rng.integers(0, RT, 3)))):
        want = pack_host(fp4[16 * t:16 * t + 16].cpu().numpy(), sc[16 * t:16 * t + 16].cpu().numpy())
        assert np.array_equal(_tile_bytes(packed, t, RT, KS, KG), want), ("tile", t)
    del packed, fp4, sc
    torch.cuda.empty_cache()
