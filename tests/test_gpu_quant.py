"""GPU quantizer and repack: bit-exact against the CPU oracle."""
import numpy as np
import pytest

import oracle
from block_scaled_precision_quant_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import block_scaled_precision_quant_amd as mx  # noqa: E402
from gpu_util import pack_host, to_dev_bf16, to_dev_u8, unpack_host  # noqa: E402


def gpu_quant(bits):
    q, s = mx.quant_a(to_dev_bf16(bits))
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("name", inputs.ORDER)
def test_quant_a_bit_exact_on_workloads(name):
    """Both operands of every workload: fp4 bytes and scale bytes identical."""
    print("case", name, flush=True)
    a, b = inputs.make(name)
    for label, x in (("A", a), ("B", b)):
        q, s = gpu_quant(x)
        rq, rs = oracle.quantize(x)
        assert np.array_equal(s, rs), (name, label, "scales")
        assert np.array_equal(q, rq), (name, label, "codes")


def coverage_matrix():
    """Groups that pair every finite bf16 magnitude with every group maximum
    at or above it: for each binade anchor (largest and a mid significand),
    the other 31 slots sweep all magnitudes up to the anchor, both signs,
    subnormals and zeros included.  Input construction only."""
    mags = np.arange(0x7F80, dtype=np.uint32)          # finite magnitudes, 0 .. max
    rows = []
    for exp in range(0, 255):
        for mant in (0x7F, 0x5F, 0x00):
            anchor = (exp << 7) | mant
            vals = mags[mags <= anchor]
            # alternate signs deterministically
            signs = ((vals * 2654435761) >> 7) & 1
            vals = (vals | (signs << 15)).astype(np.uint16)
            n = -(-vals.size // 31)
            pad = np.zeros(n * 31 - vals.size, dtype=np.uint16)
            body = np.concatenate([vals, pad]).reshape(n, 31)
            grp = np.concatenate([np.full((n, 1), anchor, dtype=np.uint16), body], axis=1)
            rows.append(grp)
    g = np.concatenate(rows)
    g = g[: g.shape[0] // 16 * 16]
    return g.reshape(-1, 512)  # 16 groups per row


def test_quant_a_exhaustive_coverage():
    x = coverage_matrix()
    print("coverage rows", x.shape, flush=True)
    q, s = gpu_quant(x)
    rq, rs = oracle.quantize(x)
    bad = np.argwhere(s != rs)
    assert bad.size == 0, ("scale", bad[:4], x.reshape(-1, 32)[bad[0][0] * 16 + bad[0][1]])
    badq = np.argwhere(q != rq)
    assert badq.size == 0, ("codes", badq[:4])


def test_quant_a_special_groups():
    """All-zero, signed-zero, saturating and tie groups, plus strided rows."""
    g = np.zeros((6, 32), dtype=np.float32)
    g[1, :] = -0.0
    g[2, 0] = 1.625  # saturates by design
    g[2, 1:] = 0.25
    g[3, :8] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]  # ties at unit scale
    g[4, :] = -3.0e38
    g[5, ::2] = 1e-40  # subnormal bf16 values, tiny scale
    bits = inputs.f32_to_bf16_bits(g.reshape(-1)).reshape(6, 32)
    bits[1, :] = 0x8000
    x = np.tile(bits.reshape(1, -1), (3, 1))  # [3, 192]
    q, s = gpu_quant(x)
    rq, rs = oracle.quantize(x)
    assert np.array_equal(s, rs) and np.array_equal(q, rq)
    # a strided view (lda > K) through the C ABI
    wide = np.zeros((3, 256), dtype=np.uint16)
    wide[:, :192] = x
    t = to_dev_bf16(wide)[:, :192]
    q2, s2 = mx.quant_a(t)
    torch.cuda.synchronize()
    assert np.array_equal(q2.cpu().numpy(), rq) and np.array_equal(s2.cpu().numpy(), rs)
    # the same groups through the packed quantizer
    buf = mx.quant_a_packed(t)
    torch.cuda.synchronize()
    assert np.array_equal(buf.cpu().numpy(), pack_host(rq, rs))


@pytest.mark.parametrize("M,K", [(1, 128), (4, 512), (17, 640), (64, 2048), (16, 7168),
                                 (5, 96), (17, 544), (1, 32)])
def test_quant_a_packed_layout(M, K):
    a, _ = inputs.make_shape(M, 16, K, seed=M + K)
    rq, rs = oracle.quantize(a)
    buf = mx.quant_a_packed(to_dev_bf16(a))
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert np.array_equal(got, pack_host(rq, rs))
    q, s = unpack_host(got, M, K)
    assert np.array_equal(q, rq) and np.array_equal(s, rs)


@pytest.mark.parametrize("M,K,lda", [(300, 2080, 2088), (33, 1056, 1064), (16, 512, 1024)])
def test_quant_a_packed_strided(M, K, lda):
    """Rows lda elements apart (a column slice of a wider matrix); ragged row
    tile, K ending inside a 128-K step and a group of four steps."""
    a, _ = inputs.make_shape(M, 16, K, seed=M + lda)
    rq, rs = oracle.quantize(a)
    wide = np.zeros((M, lda), dtype=a.dtype)
    wide[:, :K] = a
    buf = mx.quant_a_packed(to_dev_bf16(wide)[:, :K])
    torch.cuda.synchronize()
    assert np.array_equal(buf.cpu().numpy(), pack_host(rq, rs))


@pytest.mark.parametrize("N,K", [(16, 128), (2880, 512), (2112, 7168), (48, 640),
                                 (24, 96), (1, 32), (100, 544)])
def test_pack_b_layout(N, K):
    _, b = inputs.make_shape(4, N, K, seed=N)
    rq, rs = oracle.quantize(b)
    buf = mx.pack_b(to_dev_u8(rq), to_dev_u8(rs))
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert got.size == mx.packed_bytes(N, K)
    assert np.array_equal(got, pack_host(rq, rs))


@pytest.mark.parametrize("N,K", [(2880, 512), (100, 544), (7, 32)])
def test_b_prepared_from_bf16(N, K):
    """The one-time B preparation straight from bf16 (the packed quantizer
    applied to B) gives the bytes of the oracle's B, packed."""
    _, b = inputs.make_shape(1, N, K, seed=N + 3)
    rq, rs = oracle.quantize(b)
    buf = mx.quant_a_packed(to_dev_bf16(b))
    torch.cuda.synchronize()
    assert np.array_equal(buf.cpu().numpy(), pack_host(rq, rs))
