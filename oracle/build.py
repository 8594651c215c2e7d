"""Build the oracle's shared library (oracle/liboracle.so) with gcc.

Test infrastructure: the library built here is loaded only by the test suite,
the smoke check and the benchmark's CPU-baseline leg.  No fast-math and no
vector intrinsics: the oracle is meant to be read, not to be fast.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mxfp4_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(force: bool = True, out: str = LIB, src: str = SRC, extra_flags=()) -> str:
    """Compile the oracle; returns the library path.  `src` may name a
    modified copy of the source (the pin-strength test plants known mistakes
    in such copies); `extra_flags` are added to the gcc line (the sanitizer
    build)."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Wextra"] + list(extra_flags) + ["-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(force="--lazy" not in sys.argv))
