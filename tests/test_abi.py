"""C-ABI checks that need no GPU: the library loads, exports every function
include/mxfp4.h declares, and its host-side checks reject bad arguments
before anything is enqueued (every case below fails a check that precedes
all HIP calls)."""
import ctypes
import os
import re

import pytest

import block_scaled_precision_quant_amd as mx
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "mxfp4.h")

EINVAL, ENULL, EWORKSPACE, ESIZE, ENOTSUP = -1, -2, -3, -4, -5


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxfp4_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mx.library_path()):
        from block_scaled_precision_quant_amd import _build
        _build.build()
    return mx.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 12
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(mx._SIGNATURES), "binding and header disagree"


def test_version(lib):
    assert mx.version().startswith("mxfp4-gfx950")


def test_packed_bytes_closed_form(lib):
    for rows, K in [(16, 128), (4, 512), (2880, 512), (2112, 7168), (17, 640), (256, 1536),
                    (5, 32), (33, 96), (7, 544)]:
        RT, KS = -(-rows // 16), -(-K // 128)
        KG = -(-KS // 4)
        assert mx.packed_bytes(rows, K) == RT * KS * 1024 + RT * KG * 256
    # B's layout is exactly N*K/2 + N*K/32 bytes when K % 512 == 0
    assert mx.packed_bytes(2880, 512) == 2880 * 256 + 2880 * 16
    assert mx.packed_bytes(0, 512) == 0 and mx.packed_bytes(16, 100) == 0
    assert mx.packed_bytes(16, 0) == 0


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every case fails first

# The cases that pass fake device pointers must fail a host check before any
# launch; as a second guard they only run where no GPU is present.
no_gpu = pytest.mark.skipif(os.path.exists("/dev/kfd"),
                            reason="fake-pointer error-path cases run only without a GPU")


@no_gpu
def test_gemm_rejects_bad_arguments(lib):
    f = lib.mxfp4_gemm
    nb = mx.packed_bytes(32, 512)
    assert f(None, 512, FAKE, nb, FAKE, 32, 4, 32, 512, None, 0, None) == ENULL
    assert f(FAKE, 512, None, nb, FAKE, 32, 4, 32, 512, None, 0, None) == ENULL
    assert f(FAKE, 512, FAKE, nb, None, 32, 4, 32, 512, None, 0, None) == ENULL
    assert f(FAKE, 512, FAKE, nb, FAKE, 32, -1, 32, 512, None, 0, None) == EINVAL  # M
    assert f(FAKE, 512, FAKE, nb, FAKE, 32, 4, -1, 512, None, 0, None) == EINVAL   # N
    assert f(FAKE, 512, FAKE, nb, FAKE, 32, 4, 32, 500, None, 0, None) == EINVAL  # K % 32
    assert f(FAKE, 256, FAKE, nb, FAKE, 32, 4, 32, 512, None, 0, None) == EINVAL  # lda < K
    assert f(FAKE, 516, FAKE, nb, FAKE, 32, 4, 32, 512, None, 0, None) == EINVAL  # lda % 8
    assert f(FAKE, 512, FAKE, nb, FAKE, 16, 4, 32, 512, None, 0, None) == EINVAL  # ldc < N
    assert "ldc" in mx.load().mxfp4_last_error().decode()
    odd = ctypes.c_void_p(0x10008)
    assert f(odd, 512, FAKE, nb, FAKE, 32, 4, 32, 512, None, 0, None) == EINVAL  # alignment
    assert f(FAKE, 512, FAKE, nb - 1, FAKE, 32, 4, 32, 512, None, 0, None) == ESIZE


def test_empty_calls_return_at_once(lib):
    """M = 0 or N = 0 is an empty product: each entry point returns 0 before
    it reads a pointer or launches anything (so NULL pointers pass, and this
    is safe with or without a GPU).  K must still be a positive multiple of
    32 and sizes below zero are refused; an empty shape has no plan and needs
    no workspace."""
    K = 512
    for M, N in ((0, 32), (4, 0), (0, 0)):
        assert lib.mxfp4_gemm(None, 0, None, 0, None, 0, M, N, K, None, 0, None) == 0
        assert lib.mxfp4_gemm_ex(None, 0, None, 0, None, 0, M, N, K, None, 0, None, None) == 0
        assert lib.mxfp4_gemm_noalloc(None, 0, None, 0, None, 0, M, N, K, None) == 0
        assert lib.mxfp4_gemm_prequant(None, 0, None, 0, None, 0, M, N, K, None, 0, None,
                                       None) == 0
        assert lib.mxfp4_gemm_workspace_bytes(M, N, K) == 0
        assert lib.mxfp4_gemm_prequant_workspace_bytes(None, M, N, K) == 0
        assert lib.mxfp4_default_plan(M, N, K, ctypes.byref(mx._CPlan())) == EINVAL
    assert lib.mxfp4_quant_a(None, 0, K, 0, None, 0, None, 0, None) == 0
    assert lib.mxfp4_quant_a_packed(None, 0, K, 0, None, 0, None) == 0
    assert lib.mxfp4_pack_b(None, None, 0, K, None, 0, None) == 0
    assert lib.mxfp4_packed_bytes(0, K) == 0
    # an empty call with a bad K or a negative size is an error like any other
    nb = mx.packed_bytes(32, 512)
    assert lib.mxfp4_gemm(FAKE, 512, FAKE, nb, FAKE, 32, 0, 32, 500, None, 0, None) == EINVAL
    assert b"K must be" in lib.mxfp4_last_error()
    assert lib.mxfp4_gemm(FAKE, 512, FAKE, nb, FAKE, 32, -1, 0, 512, None, 0, None) == EINVAL
    assert lib.mxfp4_quant_a(FAKE, 0, 0, 512, FAKE, 256, FAKE, 16, None) == EINVAL
    assert lib.mxfp4_quant_a(FAKE, -1, 512, 512, FAKE, 256, FAKE, 16, None) == EINVAL
    assert b"M must be >= 0" in lib.mxfp4_last_error()
    assert lib.mxfp4_quant_a_packed(FAKE, 0, 500, 512, FAKE, 1 << 20, None) == EINVAL
    assert lib.mxfp4_pack_b(FAKE, FAKE, 0, 16, FAKE, 1 << 20, None) == EINVAL
    assert lib.mxfp4_pack_b(FAKE, FAKE, -2, 512, FAKE, 1 << 20, None) == EINVAL


def test_plan_checks(lib):
    M, N, K = 64, 256, 2048

    def check(plan, m=M, n=N, k=K):
        return lib.mxfp4_check_plan(ctypes.byref(plan._c()), m, n, k)

    assert check(mx.Plan(mx.MODE_PREQUANT, 4, 1, 2, 1, 16, 1)) == 0
    assert check(mx.Plan(4, 4, 1, 2, 1, 16, 1)) == EINVAL       # mode
    assert check(mx.Plan(0, 4, 1, 2, 1, 16, 1)) == EINVAL       # mode
    assert check(mx.Plan(1, 3, 1, 2, 1, 16, 1)) == ENOTSUP      # m_blocks
    assert check(mx.Plan(1, 4, 1, 2, 1, 5, 1)) == ENOTSUP       # k_steps_per_wave
    assert check(mx.Plan(1, 4, 1, 2, 1, 8, 1)) == EINVAL        # covers 8 of 16 steps
    assert check(mx.Plan(1, 1, 1, 8, 2, 8, 1)) == EINVAL        # 16 wavefronts
    # fields far out of range: refused, no overflow in the checks' products
    assert check(mx.Plan(1, 1, 1, 1 << 30, 1 << 30, 16, 1)) == EINVAL
    assert check(mx.Plan(1, 1, 1, 2, 1 << 30, 16, 1 << 30)) == EINVAL
    assert check(mx.Plan(1, 1, 1, 2, 1, 16, 0x7FFFFFFF, 2)) == EINVAL
    assert check(mx.Plan(1, 1, 1, 1, 1, 1, 16, 0)) == 0         # reduce kernel: any split
    assert check(mx.Plan(1, 1, 1, 1, 1, 1, 16, 1)) == 0         # last-WG reduce: split <= 16
    assert check(mx.Plan(1, 1, 1, 1, 1, 1, 32, 1), k=4096) == EINVAL
    assert check(mx.Plan(1, 1, 1, 1, 1, 1, 32, 0), k=4096) == 0
    assert check(mx.Plan(1, 1, 1, 1, 1, 1, 32, mx.REDUCE_ATOMIC), k=4096) == 0  # any split
    assert check(mx.Plan(1, 1, 1, 1, 1, 1, 16, 3)) == EINVAL                    # split_reduce
    assert check(mx.Plan(mx.MODE_FUSED, 1, 1, 1, 1, 4, 4, 7)) == EINVAL  # split_reduce
    # 64 rows x 128 K-steps of packed A per workgroup do not fit in LDS
    assert check(mx.Plan(mx.MODE_FUSED, 4, 1, 1, 8, 16, 1), k=16384) == EINVAL
    assert "LDS" in mx.load().mxfp4_last_error().decode()
    assert check(mx.Plan(mx.MODE_FUSED, 4, 1, 1, 1, 16, 1)) == 0
    # a dispatch holds at most 2^32 - 1 work-items: 2^32 workgroups of 64 threads
    assert check(mx.Plan(mx.MODE_FUSED, 1, 1, 1, 1, 1, 1), m=1 << 20, n=1 << 20, k=128) == EINVAL
    assert "grid too large" in mx.load().mxfp4_last_error().decode()
    # 2^17 x 2^17 with a 2-way split: the GEMM grid fits, the reduce kernel's 2^32 threads do not
    big = mx.Plan(mx.MODE_FUSED, 4, 2, 8, 1, 1, 2, mx.REDUCE_KERNEL)
    assert check(big, m=1 << 17, n=1 << 17, k=256) == EINVAL
    assert "reduce grid" in mx.load().mxfp4_last_error().decode()
    assert check(mx.Plan(*(list(big.__dict__.values())[:7] + [mx.REDUCE_LAST_WG])),
                 m=1 << 17, n=1 << 17, k=256) == 0


def test_stream_plan(lib):
    """Stream-mode plan rules: four wavefronts along N, one along K, the
    workgroup's K steps a multiple of 4, split_k the workgroups that cover K
    with them, the reduce kernel for the split; and where the default plan
    takes the mode: M <= 255, K >= 4096; any N >= 2048 from M = 96; below
    that only with two or four row blocks per workgroup and N >= 4096 (M >=
    48), N >= 7168, or K >= 8192 with N x K >= 100M; at M <= 16 only against
    a large B with long K."""
    def check(p, M, N, K):
        return lib.mxfp4_check_plan(ctypes.byref(p._c()), M, N, K)
    S = mx.MODE_STREAM
    M, N, K = 64, 1024, 16384  # 128 steps, 32 chunks
    assert check(mx.Plan(S, 4, 1, 4, 1, 128, 1, 0), M, N, K) == 0
    assert check(mx.Plan(S, 4, 2, 4, 1, 32, 4, 0), M, N, K) == 0
    assert check(mx.Plan(S, 2, 1, 4, 1, 12, 11, 0), M, N, K) == 0     # 3 chunks per workgroup: 11 workgroups
    assert check(mx.Plan(S, 2, 1, 4, 1, 12, 3, 0), M, N, K) == EINVAL
    assert check(mx.Plan(S, 4, 1, 8, 1, 128, 1, 0), M, N, K) == EINVAL  # waves_n
    assert check(mx.Plan(S, 4, 1, 4, 2, 128, 1, 0), M, N, K) == EINVAL  # waves_k
    assert check(mx.Plan(S, 4, 1, 4, 1, 126, 1, 0), M, N, K) == EINVAL  # not whole chunks
    assert check(mx.Plan(S, 4, 1, 4, 1, 132, 1, 0), M, N, K) == EINVAL  # past K
    assert check(mx.Plan(S, 4, 1, 4, 1, 32, 3, 0), M, N, K) == EINVAL   # covers 96 of 128 steps
    assert check(mx.Plan(S, 4, 1, 4, 1, 32, 4, 1), M, N, K) == EINVAL   # last-workgroup reduce
    assert check(mx.Plan(S, 3, 1, 4, 1, 128, 1, 0), M, N, K) == ENOTSUP  # m_blocks
    assert check(mx.Plan(S, 4, 1, 4, 1, 4, 1 << 20, 0), 1, 1, 1 << 23) == EINVAL  # K > 2^22
    assert check(mx.Plan(S, 1, 1, 4, 1, 1 << 30, 1, 0), M, N, K) == EINVAL
    # workspace: MX-packed A, then split partials
    ws = mx.workspace_bytes(M, N, K, mx.Plan(S, 4, 1, 4, 1, 32, 4, 0))
    a = mx.packed_bytes(M, K)
    assert ws == -(-a // 256) * 256 + 4 * M * N * 4
    assert mx.prequant_workspace_bytes(M, N, K, mx.Plan(S, 4, 1, 4, 1, 32, 4, 0)) == 4 * M * N * 4
    # the default plan
    for shape in [(64, 16384, 16384), (32, 16384, 4096), (128, 8192, 8192), (96, 4096, 14336),
                  (32, 8192, 28672), (255, 16384, 16384), (20, 12288, 12288), (17, 16384, 8192),
                  (24, 16384, 4096), (96, 4096, 4096), (160, 2560, 10240), (80, 4096, 14336),
                  (36, 5120, 20480), (16, 16384, 16384), (8, 12288, 12288), (16, 8192, 28672),
                  (256, 4096, 11008), (512, 3072, 12288), (320, 6144, 6144), (256, 8192, 8192)]:
        p = mx.default_plan(*shape)
        assert p.mode == S, (shape, p)
        mx.check_plan(p, *shape)
    for shape in [(32, 8192, 8192), (56, 5120, 5120), (40, 4096, 4096), (64, 2048, 16384),
                  (256, 16384, 16384), (64, 16384, 2048), (16, 2112, 7168), (64, 7168, 2048),
                  (8, 16384, 8192), (14, 8192, 16384), (12, 4096, 14336), (4, 16384, 16384),
                  (96, 1024, 16384), (384, 12288, 4096), (448, 7168, 7168), (256, 16384, 16384),
                  (513, 4096, 8192), (320, 7168, 7168), (384, 4096, 11008)]:
        assert mx.default_plan(*shape).mode != S, shape
    # the tiling: as many row blocks as M needs up to four, fewer while that
    # needs a split with K < 20480; two tiles per wavefront from 65 rows
    assert (mx.default_plan(64, 16384, 16384).m_blocks, mx.default_plan(64, 16384, 16384).n_tiles_per_wave) == (4, 1)
    assert (mx.default_plan(128, 16384, 16384).m_blocks, mx.default_plan(128, 16384, 16384).n_tiles_per_wave) == (4, 2)
    assert mx.default_plan(128, 8192, 8192).m_blocks == 4 and mx.default_plan(128, 8192, 8192).split_k == 1
    p = mx.default_plan(80, 4096, 14336)  # four row blocks would need a split
    assert (p.m_blocks, p.split_k) == (2, 1)
    p = mx.default_plan(96, 2048, 16384)  # so would two
    assert (p.m_blocks, p.split_k) == (1, 1)
    assert mx.default_plan(64, 4096, 14336).mode != S  # one row block below M = 96
    p = mx.default_plan(36, 5120, 20480)  # K >= 20480: keeps four row blocks and splits K
    assert (p.m_blocks, p.split_k) == (4, 3)


def test_small_m_rule(lib):
    """Small M against a B with long K, where the stream mode is not taken,
    the default plan is the fused kernel with eight wavefronts along N and K
    split over workgroups: up to 16 rows with K >= 8192 and N x K >= 100M, or
    K >= 14336 and N x K >= 30M; 17..32 rows with N <= 4096, K >= 8192 and
    N x K >= 30M."""
    for M, N, K in [(1, 16384, 16384), (4, 12288, 12288), (4, 8192, 28672), (2, 16384, 8192),
                    (12, 16384, 8192), (8, 2048, 16384), (1, 4096, 14336), (24, 4096, 14336),
                    (32, 4096, 8192), (20, 2048, 16384)]:
        p = mx.default_plan(M, N, K)
        assert (p.mode, p.m_blocks, p.waves_n, p.waves_k) == (mx.MODE_FUSED, 1, 8, 1), (M, N, K, p)
        assert p.k_steps_per_wave in (16, 14, 12, 8) and p.split_reduce == mx.REDUCE_KERNEL
        assert p.split_k * p.k_steps_per_wave == -(-K // 128)
        mx.check_plan(p, M, N, K)


def test_tiled_plan(lib):
    # the tiled mode has a fixed tiling: waves_n picks the width and split_k
    # (with split_reduce) the workgroups along K; the other fields are not
    # checked
    M, N, K = 300, 520, 640  # 5 K steps
    for fields in [(1, 1, 1, 1, 1), (0, 0, 0, 0, 0), (3, 7, 99, -1, 5)]:
        p = mx.Plan(mx.MODE_TILED, *fields, 1, 9)
        assert lib.mxfp4_check_plan(ctypes.byref(p._c()), M, N, K) == 0
        # workspace: the MX-packed A only, nothing to zero-fill; none when A
        # comes pre-quantized
        assert mx.workspace_bytes(M, N, K, p) == (mx.packed_bytes(M, K) + 255) // 256 * 256
        assert mx.workspace_zero_bytes(M, N, K, p) == 0
        assert mx.prequant_workspace_bytes(M, N, K, p) == 0
    # split of K: whole groups of four steps per workgroup, none empty, the
    # reduce kernel; the workspace adds the fp32 partials
    def check(split, reduce=0, shape=(M, N, K)):
        p = mx.Plan(mx.MODE_TILED, 1, 1, 4, 1, 1, split, reduce)
        return lib.mxfp4_check_plan(ctypes.byref(p._c()), *shape)
    assert check(2) == 0                      # steps 0-3 and 4
    assert check(3) == EINVAL                 # 5 steps hold two groups of four
    assert check(0) == EINVAL
    assert check(2, mx.REDUCE_LAST_WG) == EINVAL
    assert check(2, mx.REDUCE_ATOMIC) == EINVAL
    assert check(4, 0, (300, 520, 3072)) == EINVAL   # 24 steps in ranges of 8: the 4th is empty
    assert "without K steps" in mx.load().mxfp4_last_error().decode()
    assert check(3, 0, (300, 520, 3072)) == 0
    assert check(8, 0, (300, 520, 4096)) == 0        # 32 steps: ranges of 4
    # 2^20 tiles of 256 x 256 times a split of 8192 (K = 2^22) is 2^33
    # workgroups, past 2^32 work-items: refused
    assert check(8192, 0, (1 << 18, 1 << 18, 1 << 22)) == EINVAL
    assert "grid too large" in mx.load().mxfp4_last_error().decode()
    p = mx.Plan(mx.MODE_TILED, 1, 1, 2, 1, 1, 2, 0)
    a = (mx.packed_bytes(M, K) + 255) // 256 * 256
    assert mx.workspace_bytes(M, N, K, p) == 2 * M * N * 4 + a
    assert mx.prequant_workspace_bytes(M, N, K, p) == 2 * M * N * 4
    assert mx.workspace_zero_bytes(M, N, K, p) == 0
    # 2^20 x 2^19 is 2^23 tiles of 512 threads: one work-item more than a
    # dispatch holds; one tile column fewer fits.  The 256 x 128 tiles
    # (waves_n == 2) also have 512 threads: half the columns fit.
    p = mx.Plan(mx.MODE_TILED, 1, 1, 1, 1, 1, 1)
    assert lib.mxfp4_check_plan(ctypes.byref(p._c()), 1 << 20, 1 << 19, 128) == EINVAL
    assert "grid too large" in mx.load().mxfp4_last_error().decode()
    assert lib.mxfp4_check_plan(ctypes.byref(p._c()), 1 << 20, (1 << 19) - 256, 128) == 0
    p128 = mx.Plan(mx.MODE_TILED, 1, 1, 2, 1, 1, 1)
    assert lib.mxfp4_check_plan(ctypes.byref(p128._c()), 1 << 20, 1 << 18, 128) == EINVAL
    assert lib.mxfp4_check_plan(ctypes.byref(p128._c()), 1 << 20, (1 << 18) - 128, 128) == 0
    # buffer offsets are 32-bit: K is limited to 2^22
    assert lib.mxfp4_check_plan(ctypes.byref(p._c()), 16, 16, 1 << 22) == 0
    assert lib.mxfp4_check_plan(ctypes.byref(p._c()), 16, 16, (1 << 22) + 32) == EINVAL
    assert "K <=" in mx.load().mxfp4_last_error().decode()


@no_gpu
def test_gemm_rejects_bad_workspace(lib):
    f = lib.mxfp4_gemm_ex
    M, N, K = 64, 256, 2048
    nb = mx.packed_bytes(N, K)

    def call(plan, ws=None, wsb=0):
        cp = plan._c()
        return f(FAKE, K, FAKE, nb, FAKE, N, M, N, K, ws, wsb, ctypes.byref(cp), None)

    good = mx.Plan(mx.MODE_PREQUANT, 4, 1, 2, 1, 16, 1)
    need = mx.workspace_bytes(M, N, K, good)
    assert need == (mx.packed_bytes(M, K) + 255) // 256 * 256
    assert call(good, None, 0) == ENULL                     # workspace required
    assert call(good, FAKE, need - 1) == EWORKSPACE
    assert call(good, ctypes.c_void_p(0x10010), need) == EINVAL  # 256-byte alignment
    assert call(mx.Plan(4, 4, 1, 2, 1, 16, 1)) == EINVAL       # an invalid plan is refused
    tiled = mx.Plan(mx.MODE_TILED, 1, 1, 1, 1, 1, 1)
    assert call(tiled, None, 0) == ENULL                    # tiled: A is quantized into it
    assert call(tiled, FAKE, need - 1) == EWORKSPACE
    split = mx.Plan(mx.MODE_FUSED, 1, 1, 1, 1, 4, 4, mx.REDUCE_LAST_WG)
    assert call(split, FAKE, 256 + 4 * M * N * 4 - 4) == EWORKSPACE


def test_workspace_sizes(lib):
    M, N, K = 64, 256, 2048
    split = mx.Plan(mx.MODE_FUSED, 1, 1, 1, 1, 4, 4, mx.REDUCE_LAST_WG)
    tiles = 4 * 16  # (64/16)/1 row groups x (256/16)/1 column groups
    assert mx.workspace_zero_bytes(M, N, K, split) == 256 == -(-tiles * 4 // 256) * 256
    assert mx.workspace_bytes(M, N, K, split) == 256 + 4 * M * N * 4
    split_k = mx.Plan(mx.MODE_FUSED, 1, 1, 1, 1, 4, 4, mx.REDUCE_KERNEL)
    assert mx.workspace_zero_bytes(M, N, K, split_k) == 0
    assert mx.workspace_bytes(M, N, K, split_k) == 4 * M * N * 4
    pq = mx.Plan(mx.MODE_PREQUANT, 1, 1, 1, 1, 4, 4, mx.REDUCE_LAST_WG)
    assert mx.workspace_bytes(M, N, K, pq) == 256 + (mx.packed_bytes(M, K) + 255) // 256 * 256 \
        + 4 * M * N * 4
    assert mx.prequant_workspace_bytes(M, N, K, pq) == 256 + 4 * M * N * 4
    # atomic reduce: one zeroed [M][N] fp32 accumulator after the counters
    at = mx.Plan(mx.MODE_FUSED, 1, 1, 1, 1, 4, 4, mx.REDUCE_ATOMIC)
    assert mx.workspace_zero_bytes(M, N, K, at) == 256 + M * N * 4
    assert mx.workspace_bytes(M, N, K, at) == 256 + M * N * 4
    atq = mx.Plan(mx.MODE_PREQUANT, 1, 1, 1, 1, 4, 4, mx.REDUCE_ATOMIC)
    assert mx.workspace_bytes(M, N, K, atq) == 256 + M * N * 4 + \
        (mx.packed_bytes(M, K) + 255) // 256 * 256
    assert mx.workspace_zero_bytes(M, N, K, atq) == 256 + M * N * 4
    # without a split the reduce mode needs nothing
    one = mx.Plan(mx.MODE_FUSED, 1, 1, 1, 1, 16, 1, mx.REDUCE_ATOMIC)
    assert mx.workspace_bytes(M, N, K, one) == 0 == mx.workspace_zero_bytes(M, N, K, one)


@no_gpu
def test_quant_and_pack_reject_bad_arguments(lib):
    q = lib.mxfp4_quant_a
    assert q(None, 4, 512, 512, FAKE, 256, FAKE, 16, None) == ENULL
    assert q(FAKE, -4, 512, 512, FAKE, 256, FAKE, 16, None) == EINVAL  # M
    assert q(FAKE, 4, 48, 48, FAKE, 24, FAKE, 2, None) == EINVAL      # K % 32
    assert q(FAKE, 4, 512, 512, FAKE, 128, FAKE, 16, None) == EINVAL  # ld_fp4 < K/2
    assert q(FAKE, 4, 512, 512, FAKE, 256, FAKE, 8, None) == EINVAL   # ld_scale < K/32
    qp = lib.mxfp4_quant_a_packed
    assert qp(FAKE, 4, 512, 512, FAKE, mx.packed_bytes(4, 512) - 1, None) == ESIZE
    assert qp(FAKE, 4, 100, 104, FAKE, 1 << 20, None) == EINVAL       # K % 32
    pb = lib.mxfp4_pack_b
    assert pb(FAKE, FAKE, -1, 512, FAKE, 1 << 20, None) == EINVAL     # N
    assert pb(FAKE, FAKE, 32, 512, FAKE, mx.packed_bytes(32, 512) - 1, None) == ESIZE
    assert pb(FAKE, None, 32, 512, FAKE, 1 << 20, None) == ENULL


def test_default_plans_are_valid(lib):
    from block_scaled_precision_quant_amd import inputs
    shapes = [(w.M, w.N, w.K) for w in inputs.WORKLOADS.values()]
    shapes += [(8, 2112, 7168), (16, 3072, 1536), (64, 3072, 1536), (256, 2880, 512),
               (1, 16, 128), (100, 1008, 1152), (33, 528, 640), (1, 1, 32), (5, 24, 96),
               (70, 100, 544), (3, 4100, 8192)]
    for M, N, K in shapes:
        p = mx.default_plan(M, N, K)
        mx.check_plan(p, M, N, K)
        assert p.split_k * p.waves_k * p.k_steps_per_wave == -(-K // 128), (M, N, K, p)
        # a valid plan has a well-defined workspace size (0 only if none needed)
        ws = mx.workspace_bytes(M, N, K, p)
        if p.mode == mx.MODE_PREQUANT or p.split_k > 1:
            assert ws > 0
        assert ws == mx.workspace_bytes(M, N, K)


def test_default_plans_valid_on_random_shapes(lib):
    """The plan search returns a plan the plan rules accept for any shape a
    plan exists for: random M, N, K over the ranges callers use, plus shapes
    near the size limits where grids and the reduce kernel's thread count
    rule candidates out."""
    import numpy as np
    rng = np.random.default_rng(2024)
    shapes = [(int(rng.integers(1, 4097)), int(rng.integers(1, 65537)), 32 * int(rng.integers(1, 1025)))
              for _ in range(300)]
    shapes += [(1 << 17, 1 << 17, 256), (1, 1 << 30, 1024), (1 << 24, 16, 65536), (3, 7, 2080)]
    # a 2^20 x 2^20 C needs more than 2^32 - 1 work-items in every plan (one
    # lane covers at most one 16-row block of one column): refused, not launched
    with pytest.raises(mx.Mxfp4Error, match="grid too large"):
        mx.check_plan(mx.default_plan(1 << 20, 1 << 20, 32), 1 << 20, 1 << 20, 32)
    for M, N, K in shapes:
        p = mx.default_plan(M, N, K)
        mx.check_plan(p, M, N, K)
        if p.mode == mx.MODE_STREAM:  # whole chunks of four steps per workgroup
            kg = -(-(-(-K // 128)) // 4)
            assert p.k_steps_per_wave % 4 == 0 and p.split_k == -(-kg // (p.k_steps_per_wave // 4)), (M, N, K, p)
        elif p.mode != mx.MODE_TILED:  # the tiled mode's tiling is fixed
            assert p.split_k * p.waves_k * p.k_steps_per_wave == -(-K // 128), (M, N, K, p)
        assert mx.workspace_bytes(M, N, K) == mx.workspace_bytes(M, N, K, p)
        assert mx.default_plan(M, N, K) == p  # cached pick is the same


def test_default_plan_mode_by_size(lib):
    """Small and mid shapes keep the 16x16x128 kernels; shapes with dozens of
    256-row tiles or more go to the tiled kernel, which measured faster there
    (1.2x at 1024x4096x4096, 4x at 8192^3): 256 x 128 tiles while 256 x 256
    ones would leave CUs idle (1024x8192x8192: 128 of them), 256 x 256 from
    a full round of those on."""
    for M, N, K in [(4, 2880, 512), (256, 3072, 1536), (64, 65536, 4096), (1024, 1024, 1024)]:
        assert mx.default_plan(M, N, K).mode != mx.MODE_TILED, (M, N, K)
    for M, N, K, wide in [(1024, 4096, 4096, False), (640, 8192, 4096, False), (1536, 4096, 2048, False),
                          (1024, 8192, 8192, False), (2048, 4096, 4096, False),
                          # measured 17.9 vs 19.7 and 26.5 vs 33.3 us against the best other plans
                          (384, 6144, 2048, False), (2048, 1024, 4096, False),
                          (4096, 4096, 4096, True), (8192, 8192, 8192, True)]:
        p = mx.default_plan(M, N, K)
        assert p.mode == mx.MODE_TILED and (p.waves_n != 2) == wide, (M, N, K, p)
        assert mx.workspace_bytes(M, N, K) == mx.packed_bytes(M, K) + (-mx.packed_bytes(M, K) % 256)
    # few tiles and a long K: K split over workgroups (measured 0.53-0.94 of
    # the whole-K tiled plan's time on 18 such shapes)
    for M, N, K in [(256, 8192, 28672), (256, 5120, 20480), (640, 2048, 8192), (1024, 3072, 12288)]:
        p = mx.default_plan(M, N, K)
        assert p.mode == mx.MODE_TILED and p.split_k > 1 and p.split_reduce == mx.REDUCE_KERNEL, (M, N, K, p)
        assert mx.workspace_bytes(M, N, K) > mx.packed_bytes(M, K) + p.split_k * M * N * 4 - 1


def test_noalloc_refuses_shapes_beyond_its_scratch(lib):
    """A shape whose default plan needs more scratch than the library's
    per-GPU array is refused before any device call (so this runs on the
    CPU); fake, aligned pointers are never dereferenced."""
    cap = lib.mxfp4_gemm_noalloc_max_scratch_bytes()
    assert cap == 16 << 20
    M, N, K = 4096, 8192, 8192  # tiled plan: 17,825,792 bytes of pre-quantized A
    assert lib.mxfp4_gemm_workspace_bytes(M, N, K) > cap
    a, bp, c = 0x10000, 0x20000, 0x30000
    rc = lib.mxfp4_gemm_noalloc(a, K, bp, mx.packed_bytes(N, K), c, N, M, N, K, None)
    assert rc == EWORKSPACE
    assert b"mxfp4_gemm with a workspace" in lib.mxfp4_last_error()
    # a tiled plan that splits K keeps fp32 partials of every split: at
    # 256x8192x28672 (split 4) 32 MiB of them, beyond the array as well
    M, N, K = 256, 8192, 28672
    p = mx.default_plan(M, N, K)
    assert p.mode == mx.MODE_TILED and p.split_k > 1
    assert lib.mxfp4_gemm_workspace_bytes(M, N, K) > cap
    assert lib.mxfp4_gemm_noalloc(a, K, bp, mx.packed_bytes(N, K), c, N, M, N, K, None) == EWORKSPACE
    M, N, K = 4096, 8192, 8192
    # argument errors come first, as for mxfp4_gemm
    assert lib.mxfp4_gemm_noalloc(None, K, bp, mx.packed_bytes(N, K), c, N, M, N, K, None) == ENULL
    assert lib.mxfp4_gemm_noalloc(a, K, bp, 16, c, N, 16, N, K, None) == ESIZE
