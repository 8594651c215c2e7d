"""Build tests/c_abi_check (a plain C99 program) from tests/c_abi_check.c.

Test infrastructure: the program includes include/mxfp4.h as C, links
libmxfp4.so, the oracle's liboracle.so and the HIP runtime, and finds the two
libraries next to the repository copy it sits in (rpath relative to the
program), so it runs unchanged wherever the tree is copied.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_check.c")
EXE = os.path.join(HERE, "c_abi_check")
PKG = os.path.join(ROOT, "block_scaled_precision_quant_amd")
ORACLE = os.path.join(ROOT, "oracle")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out: str = EXE) -> str:
    """Compile with every warning an error (-pedantic for the library's own
    header; the HIP headers are system headers); returns the program path."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-pedantic"] + [
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-isystem", os.path.join(ROCM, "include"), SRC, "-o", tmp,
           "-L", PKG, "-lmxfp4", "-L", ORACLE, "-loracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../block_scaled_precision_quant_amd:$ORIGIN/../oracle:"
           + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("gcc failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
