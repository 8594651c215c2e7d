"""The Python binding refuses, before any pointer reaches the library, tensors
that the C functions cannot check themselves: host tensors and non-tensors
(CPU only: these checks come before the library is touched)."""
import pytest

torch = pytest.importorskip("torch")
import block_scaled_precision_quant_amd as mx  # noqa: E402


def test_host_tensors_are_refused():
    a = torch.zeros((4, 512), dtype=torch.bfloat16)
    u8 = torch.zeros(1024, dtype=torch.uint8)
    calls = {
        "gemm": lambda: mx.gemm(a, u8, 64),
        "gemm_noalloc": lambda: mx.gemm_noalloc(a, u8, 64, out=torch.empty((4, 64), dtype=torch.bfloat16)),
        "gemm_prequant": lambda: mx.gemm_prequant(u8, 4, u8, 64, 512),
        "quant_a": lambda: mx.quant_a(a),
        "quant_a_packed": lambda: mx.quant_a_packed(a),
        "pack_b": lambda: mx.pack_b(torch.zeros((64, 256), dtype=torch.uint8),
                                    torch.zeros((64, 16), dtype=torch.uint8)),
    }
    for name, call in calls.items():
        with pytest.raises(ValueError, match="must be on a GPU"):
            call()


def test_non_tensors_are_refused():
    with pytest.raises(TypeError, match="must be a torch.Tensor"):
        mx.gemm([[0.0] * 512] * 4, None, 64)
    with pytest.raises(TypeError, match="must be a torch.Tensor"):
        mx.pack_b(b"\0" * 64, b"\0" * 4)
