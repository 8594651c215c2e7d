"""Helpers for the GPU tests: host <-> device moves and the MX-packed layout
written out from its closed form in include/mxfp4.h (numpy, host side)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")


def dev():
    return torch.device("cuda:0")


def to_dev_bf16(bits):
    """uint16 bf16 bit array -> CUDA bfloat16 tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev()).view(torch.bfloat16)


def to_dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev())


def bf16_out_to_f32(c):
    """CUDA bf16 tensor -> float32 numpy (exact widening)."""
    return c.float().cpu().numpy()


def packed_dims(rows, K):
    RT = -(-rows // 16)
    KS = -(-K // 128)
    KG = -(-KS // 4)
    return RT, KS, KG


def pack_host(fp4, scale):
    """Linear fp4x2 [R, K/2] + e8m0 [R, K/32] -> MX-packed bytes (padding rows
    and K-groups past K: code 0, scale 127; scale bytes of steps >= KS: 127)."""
    R, half = fp4.shape
    K = 2 * half
    RT, KS, KG = packed_dims(R, K)
    q = np.zeros((RT * 16, KS * 64), dtype=np.uint8)
    q[:R, :half] = fp4
    s = np.full((RT * 16, KG * 16), 127, dtype=np.uint8)
    s[:R, :K // 32] = scale
    # data[t, j, h, r, i] = q[16t + r, 64j + 16h + i]
    data = q.reshape(RT, 16, KS, 4, 16).transpose(0, 2, 3, 1, 4).reshape(-1)
    # sc[t, g, h, r, s] = scale[16t + r, 4*(4g + s) + h]
    sc = s.reshape(RT, 16, KG, 4, 4).transpose(0, 2, 4, 1, 3).reshape(-1)
    return np.concatenate([data, sc])


def unpack_host(buf, R, K):
    """Inverse of pack_host: MX-packed bytes -> (fp4 [R, K/2], scale [R, K/32])."""
    RT, KS, KG = packed_dims(R, K)
    D = RT * KS * 1024
    data = np.asarray(buf[:D], dtype=np.uint8).reshape(RT, KS, 4, 16, 16)
    q = data.transpose(0, 3, 1, 2, 4).reshape(RT * 16, KS * 64)
    sc = np.asarray(buf[D:D + RT * KG * 256], dtype=np.uint8).reshape(RT, KG, 4, 16, 4)
    s = sc.transpose(0, 3, 1, 4, 2).reshape(RT * 16, KG * 16)
    return q[:R, :K // 2], s[:R, :K // 32]


def assert_close_to_oracle(got, want, label=""):
    """Elementwise |got - want| <= 1e-2*|want| + 1e-2 (want: oracle fp32)."""
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    tol = 1e-2 * np.abs(want.astype(np.float64)) + 1e-2
    bad = np.argwhere(~(err <= tol))
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError("%s: %d of %d outside tolerance; first at %s: got %r want %r"
                             % (label, len(bad), got.size, i, float(got[i]), float(want[i])))
