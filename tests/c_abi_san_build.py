"""Sanitizer build of the C-ABI check (CPU only; test infrastructure).

Builds, into a directory of the caller's choosing:

* libmxfp4.so whose host code (api.cpp: argument checks, plans, workspace
  layout) is compiled with AddressSanitizer and UndefinedBehaviorSanitizer,
  linked with the kernel objects of the normal build (_build/*.o; the GPU
  code itself is not instrumented: every sanitizer flag is host-only);
* tests/c_abi_check.c, compiled by the same clang with the same sanitizers,
  linked against that library.

Both sides use clang's shared sanitizer runtime, so one runtime serves the
program and the library.  No GPU is needed for the program's `host` mode.
"""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "block_scaled_precision_quant_amd")
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
ORACLE = os.path.join(ROOT, "oracle")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
KERNEL_OBJECTS = ["gemm.o", "gemm_tiled.o", "quant.o"]

# host-only: each sanitizer option goes to the host pass alone
HOST_SAN = []
for _flag in ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer"]:
    HOST_SAN += ["-Xarch_host", _flag]


def tools():
    """(hipcc, clang, directory of clang's sanitizer runtimes) or None."""
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    rt = glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                "libclang_rt.asan-x86_64.so"))
    if not (os.path.exists(hipcc) and os.path.exists(clang) and rt):
        return None
    return hipcc, clang, os.path.dirname(rt[0])


def kernel_objects():
    objs = [os.path.join(BUILD, o) for o in KERNEL_OBJECTS]
    return objs if all(os.path.exists(o) for o in objs) else None


def _run(cmd, what):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("%s failed:\n%s\n%s" % (what, " ".join(cmd), r.stderr[-4000:]))


def build(out_dir: str) -> str:
    """Builds the sanitized library and program in out_dir; returns the
    program's path.  Requires tools() and kernel_objects()."""
    hipcc, clang, rt_dir = tools()
    objs = kernel_objects()
    api_obj = os.path.join(out_dir, "api_san.o")
    _run([hipcc, "-x", "hip", "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include")] + HOST_SAN +
         ["-c", os.path.join(CSRC, "api.cpp"), "-o", api_obj], "hipcc (api.cpp)")
    lib = os.path.join(out_dir, "libmxfp4.so")
    _run([hipcc, "-shared", "-fPIC", "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", lib, api_obj] + objs,
         "link (libmxfp4.so)")
    exe = os.path.join(out_dir, "c_abi_check_san")
    _run([clang, "-std=c99", "-O1", "-g", "-Wall", "-Wextra", "-Werror", "-pedantic",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          "-shared-libsan", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
          "-isystem", os.path.join(ROCM, "include"), os.path.join(HERE, "c_abi_check.c"),
          "-o", exe, "-L", out_dir, "-lmxfp4", "-L", ORACLE, "-loracle",
          "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
          "-Wl,-rpath," + ":".join([out_dir, ORACLE, os.path.join(ROCM, "lib"), rt_dir])],
         "clang (c_abi_check.c)")
    return exe
