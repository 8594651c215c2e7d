"""MXFP4 GEMM for MI355X (gfx950): Python binding of libmxfp4.so.

C[M, N] = A[M, K] . B[N, K]^T with bf16 output; A is bf16 and quantized on the
fly to MXFP4 (e2m1 codes, one e8m0 scale per 32 K-elements), B is quantized
once and repacked into the kernels' layout.

This module only marshals arguments: tensors become device pointers, the
current torch stream becomes the HIP stream, and every computation runs in
the library's HIP kernels.  There is no fallback path: if the library is
missing or a call fails, an exception is raised.  The C functions and their
contracts are declared in include/mxfp4.h.

Before a pointer is passed on, each tensor is checked for what the C
functions cannot see: that it lives on a GPU, its dtype, and a shape and
strides whose memory covers everything the call reads or writes (a tensor
that fails raises TypeError or ValueError and nothing is launched).
"""
import ctypes
import os
from dataclasses import dataclass

__all__ = [
    "Mxfp4Error", "Plan", "MODE_FUSED", "MODE_PREQUANT", "MODE_TILED", "MODE_STREAM", "REDUCE_KERNEL",
    "REDUCE_LAST_WG",
    "REDUCE_ATOMIC", "library_path", "load", "packed_bytes",
    "pack_b", "quant_a", "quant_a_packed", "default_plan", "check_plan", "workspace_bytes", "workspace_zero_bytes",
    "prequant_workspace_bytes", "new_workspace", "gemm", "gemm_noalloc", "noalloc_max_scratch_bytes",
    "gemm_prequant", "version",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
MODE_FUSED = 1
MODE_PREQUANT = 2
MODE_TILED = 3  # 32x32x64 instruction; waves_n == 2: 256 x 128 tiles, else 256 x 256; other fields ignored
MODE_STREAM = 4  # K loop inside the workgroup: waves_n 4, waves_k 1, k_steps_per_wave = steps per workgroup
REDUCE_KERNEL = 0
REDUCE_LAST_WG = 1
REDUCE_ATOMIC = 2

_ERR_NAMES = {-1: "EINVAL", -2: "ENULL", -3: "EWORKSPACE", -4: "ESIZE", -5: "ENOTSUP", -6: "EHIP"}


class Mxfp4Error(RuntimeError):
    def __init__(self, code, message):
        super().__init__("mxfp4 %s (%d): %s" % (_ERR_NAMES.get(code, "?"), code, message))
        self.code = code


class _CPlan(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int), ("m_blocks", ctypes.c_int),
                ("n_tiles_per_wave", ctypes.c_int), ("waves_n", ctypes.c_int),
                ("waves_k", ctypes.c_int), ("k_steps_per_wave", ctypes.c_int),
                ("split_k", ctypes.c_int), ("split_reduce", ctypes.c_int)]


@dataclass(frozen=True)
class Plan:
    """Tiling of one GEMM call (fields as in mxfp4_plan)."""
    mode: int
    m_blocks: int
    n_tiles_per_wave: int
    waves_n: int
    waves_k: int
    k_steps_per_wave: int
    split_k: int
    split_reduce: int = 1  # REDUCE_LAST_WG

    def _c(self):
        return _CPlan(self.mode, self.m_blocks, self.n_tiles_per_wave, self.waves_n, self.waves_k,
                      self.k_steps_per_wave, self.split_k, self.split_reduce)


_LIB = None
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_i = ctypes.c_int

# name -> (restype, argtypes); every symbol the header declares
_SIGNATURES = {
    "mxfp4_packed_bytes": (_sz, [_i, _i]),
    "mxfp4_pack_b": (_i, [_vp, _vp, _i, _i, _vp, _sz, _vp]),
    "mxfp4_quant_a": (_i, [_vp, _i, _i, _i, _vp, _i, _vp, _i, _vp]),
    "mxfp4_quant_a_packed": (_i, [_vp, _i, _i, _i, _vp, _sz, _vp]),
    "mxfp4_default_plan": (_i, [_i, _i, _i, ctypes.POINTER(_CPlan)]),
    "mxfp4_check_plan": (_i, [ctypes.POINTER(_CPlan), _i, _i, _i]),
    "mxfp4_plan_workspace_bytes": (_sz, [ctypes.POINTER(_CPlan), _i, _i, _i]),
    "mxfp4_plan_workspace_zero_bytes": (_sz, [ctypes.POINTER(_CPlan), _i, _i, _i]),
    "mxfp4_gemm_workspace_bytes": (_sz, [_i, _i, _i]),
    "mxfp4_gemm_prequant_workspace_bytes": (_sz, [ctypes.POINTER(_CPlan), _i, _i, _i]),
    "mxfp4_gemm": (_i, [_vp, _i, _vp, _sz, _vp, _i, _i, _i, _i, _vp, _sz, _vp]),
    "mxfp4_gemm_ex": (_i, [_vp, _i, _vp, _sz, _vp, _i, _i, _i, _i, _vp, _sz,
                           ctypes.POINTER(_CPlan), _vp]),
    "mxfp4_gemm_noalloc": (_i, [_vp, _i, _vp, _sz, _vp, _i, _i, _i, _i, _vp]),
    "mxfp4_gemm_noalloc_max_scratch_bytes": (_sz, []),
    "mxfp4_gemm_prequant": (_i, [_vp, _sz, _vp, _sz, _vp, _i, _i, _i, _i, _vp, _sz,
                                 ctypes.POINTER(_CPlan), _vp]),
    "mxfp4_last_error": (ctypes.c_char_p, []),
    "mxfp4_version": (ctypes.c_char_p, []),
}


def library_path():
    return os.path.join(_PKG, "libmxfp4.so")


def load():
    """Load libmxfp4.so (built by __graft_entry__.build()); raises if absent."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise ImportError("libmxfp4.so is not built (%s); run __graft_entry__.build()" % path)
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def _check(rc):
    if rc != 0:
        raise Mxfp4Error(rc, load().mxfp4_last_error().decode())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _nbytes(t):
    return t.numel() * t.element_size()


def _gpu(t, name, dtype=None, like=None):
    """`t` is a GPU tensor (of `dtype`, on the device of `like` when given)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor (got %s)" % (name, type(t).__name__))
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU (got device %s)" % (name, t.device))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if like is not None and t.device != like.device:
        raise ValueError("%s is on %s, the other operands on %s" % (name, t.device, like.device))
    return t


def _flat(t, name, dtype=None, like=None):
    """A buffer passed as pointer + byte count: its bytes must be contiguous."""
    _gpu(t, name, dtype, like)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous (its size is passed in bytes)" % name)
    return t


def _matrix(t, name, dtype, rows, cols, like=None):
    """A [rows, cols] matrix with unit stride along cols; its row stride is the
    leading dimension passed on (the C functions check it against cols)."""
    _gpu(t, name, dtype, like)
    if t.dim() != 2 or tuple(t.shape) != (rows, cols):
        raise ValueError("%s must have shape (%d, %d) (got %s)" % (name, rows, cols, tuple(t.shape)))
    if cols > 1 and t.stride(1) != 1:
        raise ValueError("%s must have unit stride along its second dimension" % name)
    return t


def version():
    return load().mxfp4_version().decode()


def packed_bytes(rows, K):
    """Bytes of the MX-packed layout of `rows` x K (0 if invalid)."""
    return int(load().mxfp4_packed_bytes(int(rows), int(K)))


def pack_b(b_fp4, b_scale, out=None, stream=None):
    """Repack linear fp4x2 [N, K/2] + e8m0 [N, K/32] (uint8 CUDA tensors) into
    the MX-packed layout; returns the uint8 buffer."""
    import torch
    _flat(b_fp4, "b_fp4", torch.uint8)
    if b_fp4.dim() != 2:
        raise ValueError("b_fp4 must be 2-D [N, K/2] (got %s)" % (tuple(b_fp4.shape),))
    N, half = b_fp4.shape
    K = 2 * half
    _flat(b_scale, "b_scale", torch.uint8, like=b_fp4)
    if tuple(b_scale.shape) != (N, K // 32):
        raise ValueError("b_scale must have shape (%d, %d) (got %s)" % (N, K // 32, tuple(b_scale.shape)))
    if out is None:
        out = torch.empty(packed_bytes(N, K), dtype=torch.uint8, device=b_fp4.device)
    _flat(out, "out", like=b_fp4)
    _check(load().mxfp4_pack_b(_ptr(b_fp4), _ptr(b_scale), N, K, _ptr(out), _nbytes(out),
                               _stream(stream)))
    return out


def _rows(a):
    import torch
    _gpu(a, "a", torch.bfloat16)
    if a.dim() != 2 or (a.shape[1] > 1 and a.stride(1) != 1):
        raise ValueError("a must be a 2-D tensor with unit stride along K")
    return a.shape[0], a.shape[1], a.stride(0)


def quant_a(a, out_fp4=None, out_scale=None, stream=None):
    """Quantize bf16 [M, K] to linear fp4x2 [M, K/2] + e8m0 [M, K/32]."""
    import torch
    M, K, lda = _rows(a)
    if out_fp4 is None:
        out_fp4 = torch.empty((M, K // 2), dtype=torch.uint8, device=a.device)
    if out_scale is None:
        out_scale = torch.empty((M, K // 32), dtype=torch.uint8, device=a.device)
    _matrix(out_fp4, "out_fp4", torch.uint8, M, K // 2, like=a)
    _matrix(out_scale, "out_scale", torch.uint8, M, K // 32, like=a)
    _check(load().mxfp4_quant_a(_ptr(a), M, K, lda, _ptr(out_fp4), out_fp4.stride(0),
                                _ptr(out_scale), out_scale.stride(0), _stream(stream)))
    return out_fp4, out_scale


def quant_a_packed(a, out=None, stream=None):
    """Quantize bf16 [M, K] straight into the MX-packed layout."""
    import torch
    M, K, lda = _rows(a)
    if out is None:
        out = torch.empty(packed_bytes(M, K), dtype=torch.uint8, device=a.device)
    _flat(out, "out", like=a)
    _check(load().mxfp4_quant_a_packed(_ptr(a), M, K, lda, _ptr(out), _nbytes(out),
                                       _stream(stream)))
    return out


def default_plan(M, N, K):
    p = _CPlan()
    _check(load().mxfp4_default_plan(M, N, K, ctypes.byref(p)))
    return Plan(p.mode, p.m_blocks, p.n_tiles_per_wave, p.waves_n, p.waves_k,
                p.k_steps_per_wave, p.split_k, p.split_reduce)


def check_plan(plan, M, N, K):
    """Raise Mxfp4Error unless `plan` is valid for the shape and compiled into the library."""
    cp = plan._c()
    _check(load().mxfp4_check_plan(ctypes.byref(cp), M, N, K))


def workspace_bytes(M, N, K, plan=None):
    if plan is None:
        return int(load().mxfp4_gemm_workspace_bytes(M, N, K))
    cp = plan._c()
    return int(load().mxfp4_plan_workspace_bytes(ctypes.byref(cp), M, N, K))


def workspace_zero_bytes(M, N, K, plan=None):
    """Leading workspace bytes that must be zero before first use."""
    if plan is None and (M == 0 or N == 0):
        return 0  # an empty product needs no workspace
    p = plan if plan is not None else default_plan(M, N, K)
    cp = p._c()
    return int(load().mxfp4_plan_workspace_zero_bytes(ctypes.byref(cp), M, N, K))


def prequant_workspace_bytes(M, N, K, plan=None):
    cp = plan._c() if plan is not None else None
    return int(load().mxfp4_gemm_prequant_workspace_bytes(
        ctypes.byref(cp) if cp is not None else None, M, N, K))


def new_workspace(nbytes, device):
    """A zero-filled workspace (its tile counters start at zero)."""
    import torch
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _workspace(nbytes, device, workspace):
    if workspace is not None:
        return _flat(workspace, "workspace")
    if nbytes == 0:
        return None
    return new_workspace(nbytes, device)


def gemm(a, b_packed, N, out=None, workspace=None, plan=None, stream=None):
    """C = A . B^T: A bf16 [M, K] (CUDA), b_packed from pack_b for N rows.
    Returns bf16 [M, N] (written into `out` when given)."""
    import torch
    M, K, lda = _rows(a)
    _flat(b_packed, "b_packed", like=a)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _matrix(out, "out", torch.bfloat16, M, N, like=a)
    workspace = _workspace(workspace_bytes(M, N, K, plan), a.device, workspace)
    if workspace is not None:
        _gpu(workspace, "workspace", like=a)
    cp = plan._c() if plan is not None else None
    _check(load().mxfp4_gemm_ex(_ptr(a), lda, _ptr(b_packed), _nbytes(b_packed), _ptr(out),
                                out.stride(0), M, N, K, _ptr(workspace),
                                _nbytes(workspace) if workspace is not None else 0,
                                ctypes.byref(cp) if cp is not None else None, _stream(stream)))
    return out


def noalloc_max_scratch_bytes():
    """Bytes of the library's per-GPU scratch array used by gemm_noalloc."""
    return int(load().mxfp4_gemm_noalloc_max_scratch_bytes())


def gemm_noalloc(a, b_packed, N, out, stream=None):
    """C = A . B^T with the default plan and no workspace: the scratch lives in
    the library's per-GPU array (calls on one GPU must not overlap).  `out`
    (bf16 [M, N] or wider rows) is required, so nothing is allocated here
    either."""
    import torch
    M, K, lda = _rows(a)
    _flat(b_packed, "b_packed", like=a)
    _matrix(out, "out", torch.bfloat16, M, N, like=a)
    _check(load().mxfp4_gemm_noalloc(_ptr(a), lda, _ptr(b_packed), _nbytes(b_packed), _ptr(out),
                                     out.stride(0), M, N, K, _stream(stream)))
    return out


def gemm_prequant(a_packed, M, b_packed, N, K, out=None, workspace=None, plan=None, stream=None):
    """C = A . B^T with A already MX-packed (from quant_a_packed)."""
    import torch
    _flat(a_packed, "a_packed")
    _flat(b_packed, "b_packed", like=a_packed)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a_packed.device)
    _matrix(out, "out", torch.bfloat16, M, N, like=a_packed)
    # an empty product (M or N = 0) has no plan; the call returns at once
    p = plan if plan is not None or M == 0 or N == 0 else default_plan(M, N, K)
    workspace = _workspace(prequant_workspace_bytes(M, N, K, p), a_packed.device, workspace)
    if workspace is not None:
        _gpu(workspace, "workspace", like=a_packed)
    cp = p._c() if p is not None else None
    _check(load().mxfp4_gemm_prequant(_ptr(a_packed), _nbytes(a_packed), _ptr(b_packed),
                                      _nbytes(b_packed), _ptr(out), out.stride(0), M, N, K,
                                      _ptr(workspace),
                                      _nbytes(workspace) if workspace is not None else 0,
                                      ctypes.byref(cp) if cp is not None else None,
                                      _stream(stream)))
    return out
