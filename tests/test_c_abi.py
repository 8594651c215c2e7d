"""The C ABI used from plain C: include/mxfp4.h compiled as C99 with
-pedantic -Werror, the program linked against libmxfp4.so (tests/c_abi_check.c).

CPU: the header compiles as C and the host-only entry points (size queries,
plans, argument errors) answer as documented.  GPU: one GEMM through the HIP
runtime's C API and the library alone (B quantized by the oracle, repacked on
the GPU; A quantized inside the GEMM), checked against the oracle, and the
quantizer's bytes checked exactly.  The program is built by
__graft_entry__.build(); the CPU test rebuilds it, the GPU test runs what was
built.
"""
import importlib.util
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _builder():
    spec = importlib.util.spec_from_file_location("c_abi_build", os.path.join(HERE, "c_abi_build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_c_header_and_host_entry_points():
    exe = _builder().build()
    r = subprocess.run([exe, "host"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host checks ok" in r.stdout


@pytest.mark.gpu
def test_c_program_gemm_on_gpu():
    exe = _builder().EXE
    assert os.path.exists(exe), "tests/c_abi_check not built: run __graft_entry__.build()"
    print("c_abi_check gpu: 48 x 272 x 640", flush=True)
    r = subprocess.run([exe, "gpu"], capture_output=True, text=True, timeout=100)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "gpu check ok" in r.stdout, r.stdout
