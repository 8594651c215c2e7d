"""Ahead-of-time build of libmxfp4.so for gfx950 with hipcc.

Each source compiles to an object in _build/ (in parallel), then one shared
library is linked next to this file.  No fast-math anywhere: the quantizer
must be bit-exact.

Every kernel's resource use (registers, scratch, LDS, occupancy) comes from
the compiler's kernel-resource-usage remarks; build() writes them to
_build/kernel_resources.txt, prints a summary, and fails if any kernel
uses scratch memory or spills vector registers (a spill would otherwise show
only as a slowdown).  Scalar-register spills go to lanes of vector
registers, not to memory; they are reported, not refused.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmxfp4.so")
REPORT = os.path.join(BUILD, "kernel_resources.txt")
SOURCES = ["quant.hip", "gemm.hip", "gemm_tiled.hip", "gemm_stream.hip", "api.cpp"]
HEADERS = ["mx_device.hpp", "mx_internal.hpp"]
ARCH = "gfx950"

_REMARK = re.compile(r"remark:\s+(?:Function Name: (\S+)|([A-Za-z][A-Za-z \[\]/]*?): (\S+)) \[-Rpass-analysis")
_FIELDS = {"TotalSGPRs": "sgpr", "VGPRs": "vgpr", "AGPRs": "agpr",
           "ScratchSize [bytes/lane]": "scratch", "Occupancy [waves/SIMD]": "occupancy",
           "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill",
           "LDS Size [bytes/block]": "lds", "Dynamic Stack": "dynamic_stack"}


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else (shutil.which("hipcc") or "hipcc")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-result", "-I", os.path.join(ROOT, "include")]


def parse_resources(stderr, source):
    """Kernel records from the compiler's kernel-resource-usage remarks."""
    out, cur = [], None
    for line in stderr.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        if m.group(1):
            cur = {"source": source, "symbol": m.group(1)}
            out.append(cur)
        elif cur is not None and m.group(2) in _FIELDS:
            v = m.group(3)
            cur[_FIELDS[m.group(2)]] = v if m.group(2) == "Dynamic Stack" else int(v)
    return out


def demangle(names):
    try:
        r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True)
        out = r.stdout.splitlines()
        if r.returncode == 0 and len(out) == len(names):
            return out
    except OSError:
        pass
    return list(names)


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + ["-Rpass-analysis=kernel-resource-usage",
                                        "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj, parse_resources(r.stderr, src)


def write_report(kernels):
    """Writes the per-kernel table; raises if any kernel uses scratch memory,
    spills vector registers or needs a dynamic stack."""
    names = demangle([k["symbol"] for k in kernels])
    lines = ["# kernel resources, gfx950 (compiler remarks): source | kernel | SGPR VGPR AGPR | "
             "scratch B/lane | spills (SGPR, VGPR) | LDS B (static) | occupancy waves/SIMD"]
    bad = []
    for k, name in zip(kernels, names):
        k["name"] = name
        lines.append("%s | %s | %d %d %d | %d | %d %d | %d | %d" % (
            k["source"], name, k.get("sgpr", -1), k.get("vgpr", -1), k.get("agpr", -1),
            k.get("scratch", -1), k.get("sgpr_spill", -1), k.get("vgpr_spill", -1),
            k.get("lds", -1), k.get("occupancy", -1)))
        if (k.get("scratch", 1) != 0 or k.get("vgpr_spill", 1) != 0
                or k.get("dynamic_stack", "False") != "False"):
            bad.append(name)
    os.makedirs(BUILD, exist_ok=True)
    with open(REPORT, "w") as f:
        f.write("\n".join(lines) + "\n")
    if bad:
        raise RuntimeError("kernels using scratch memory or spilling vector registers (see %s):\n  %s"
                           % (REPORT, "\n  ".join(bad)))
    return kernels


def summary(kernels):
    vg = max(kernels, key=lambda k: k.get("vgpr", 0) + k.get("agpr", 0))
    sg = [k for k in kernels if k.get("sgpr_spill", 0)]
    return ("%d kernels, no scratch and no vector-register spills; most registers: %s "
            "(%d VGPR + %d AGPR, occupancy %d); %d spill scalar registers into vector lanes "
            "(at most %d); report: %s" % (
                len(kernels), vg["name"], vg.get("vgpr", 0), vg.get("agpr", 0),
                vg.get("occupancy", 0), len(sg), max([k["sgpr_spill"] for k in sg] or [0]),
                REPORT))


def build(jobs=None):
    """Compile every source and link libmxfp4.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    kernels = [k for _, ks in results for k in ks]
    if not kernels:
        raise RuntimeError("the compiler printed no kernel-resource-usage remarks; "
                           "cannot check the kernels for scratch use")
    kernels = write_report(kernels)
    print(summary(kernels))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    return LIB


def stale():
    """True when the library is missing or older than a source or header."""
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = [os.path.join(CSRC, f) for f in SOURCES + HEADERS]
    deps.append(os.path.join(ROOT, "include", "mxfp4.h"))
    return any(os.path.getmtime(d) > t for d in deps)


if __name__ == "__main__":
    import time
    t0 = time.time()
    print(build(), "%.1fs" % (time.time() - t0))
