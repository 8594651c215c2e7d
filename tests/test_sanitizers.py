"""Host sanitizers (CPU only): the oracle and the host side of the C ABI run
clean under AddressSanitizer and UndefinedBehaviorSanitizer.

* The oracle's C library is rebuilt with -fsanitize=address,undefined into a
  temporary file and the oracle's whole pin suite (tests/test_oracle.py,
  including the exhaustive sweeps) runs against it in a child interpreter
  with the ASan runtime preloaded (the interpreter itself is not
  instrumented); any report aborts the child.
* The plain-C ABI program (tests/c_abi_check.c) and the host code of
  libmxfp4.so (argument checks, plan search, workspace layout) are built
  with the same sanitizers by clang (tests/c_abi_san_build.py; the GPU
  kernels are linked in unchanged) and the program runs its host checks:
  size queries, plans, argument errors and out-of-range plan fields, no GPU.
"""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
from oracle import build as oracle_build  # noqa: E402

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def runtime(name):
    r = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc has no %s here" % name)
    return path


def san_env(preload):
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("a library is already preloaded in this environment; not replacing it")
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    if preload:
        env["LD_PRELOAD"] = preload
    return env


def check_clean(r):
    text = r.stdout + r.stderr
    assert "AddressSanitizer" not in text and "runtime error:" not in text, text[-4000:]
    assert r.returncode == 0, text[-4000:]


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = oracle_build.build(out=str(tmp_path / "liboracle_san.so"), extra_flags=SAN)
    env = san_env(runtime("libasan.so"))
    env["MXFP4_ORACLE_LIB"] = lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    check_clean(r)
    assert " passed" in r.stdout


def test_c_abi_host_checks_under_asan_ubsan(tmp_path):
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "c_abi_san_build", os.path.join(ROOT, "tests", "c_abi_san_build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    if mod.tools() is None:
        pytest.skip("ROCm clang or its sanitizer runtime is not installed here")
    if mod.kernel_objects() is None:
        pytest.skip("the library's kernel objects are not built (_build/); run build() first")
    exe = mod.build(str(tmp_path))
    env = san_env(None)
    env["ASAN_OPTIONS"] = "abort_on_error=1"  # leak checking on: a plain C program
    r = subprocess.run([exe, "host"], capture_output=True, text=True, timeout=120, env=env)
    check_clean(r)
    assert "host checks ok" in r.stdout
