"""Benchmark: L2-cold microseconds per MXFP4 GEMM call on one MI355X.

Default workload: the two M=32, K=512 shapes (N=4096 and N=2880).  One step
is one call of each shape; before every timed call a 512 MiB device fill
evicts the L2 caches and the Infinity Cache, and HIP events on the launch
stream bracket the call alone.  Inputs (A bf16, packed B) are resident in
HBM before timing starts; B is quantized by the library's own quantizer and
repacked once (reported separately as prepack_us).

Prints one JSON line.  `value` is the mean over the workload's shapes of the
median L2-cold event time per call (µs, lower is better).  `ms_per_step`
is wall time per step including the cache-evicting fills.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--all]
                  [--large] [--no-cpu-baseline]

--large adds one line per large shape (M >= 1024), whose default plan is the
tiled kernel: the L2-cold time per call (quantizer launch included) and the
same plan's time on pre-quantized A, each with its fraction of the dense FP4
peak.
"""
import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from block_scaled_precision_quant_amd import inputs  # noqa: E402

HBM_PEAK_GBPS = 8000.0
FP4_PEAK_TFLOPS = 10100.0
FLUSH_BYTES = 512 << 20

WORKLOAD_SETS = {
    "m32_k512": ["m32_n4096_k512", "m32_n2880_k512"],
}
for _n in inputs.ORDER:
    WORKLOAD_SETS[_n] = [_n]


def alg_bytes(M, N, K):
    """Bytes the method itself must move per call: A bf16, B fp4 + e8m0, C bf16."""
    return 2 * M * K + N * K // 2 + N * K // 32 + 2 * M * N


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="m32_k512", choices=sorted(WORKLOAD_SETS))
    ap.add_argument("--all", action="store_true", help="one extra JSON line per tuned shape")
    ap.add_argument("--large", action="store_true",
                    help="one extra JSON line per large shape (tiled 256 x 256 kernel)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 64 MiB device copy first (a known-size kernel for "
                         "scaling hardware byte counters)")
    return ap.parse_args()


# large shapes for --large: (M, N, K), seeded like the workloads
LARGE = [(1024, 8192, 8192), (4096, 4096, 4096), (8192, 8192, 8192)]

# --all also times the alternatives to the default plan where the workload
# makes a choice: the fastest pre-quantized-A plan of an L2-cold sweep over
# every valid plan (a separate quantizer launch, then the GEMM), and the
# tiled mode.  Fields: mode, m_blocks, n_tiles_per_wave, waves_n, waves_k,
# k_steps_per_wave, split_k.
ALTERNATIVES = {
    "m64_n7168_k2048": {"prequant": (2, 2, 1, 4, 2, 8, 1)},
    "m256_n3072_k1536": {"prequant": (2, 2, 1, 6, 1, 12, 1), "tiled": (3, 1, 1, 2, 1, 1, 1)},
}


class Case:
    """Device-resident inputs and outputs of one shape."""

    def __init__(self, name, torch, mx):
        w = inputs.WORKLOADS[name] if isinstance(name, str) else name
        name = w.name
        self.name, self.M, self.N, self.K = name, w.M, w.N, w.K
        a_bits, b_bits = inputs.make(w)
        dev = torch.device("cuda:0")
        to = lambda bits: torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
        self.a = to(a_bits)
        b = to(b_bits)
        self.bq, self.bs = mx.quant_a(b)  # the library's quantizer on B's rows
        self.b_packed = torch.empty(mx.packed_bytes(self.N, self.K), dtype=torch.uint8, device=dev)
        self.c = torch.empty((self.M, self.N), dtype=torch.bfloat16, device=dev)
        self.plan = mx.default_plan(self.M, self.N, self.K)
        nws = mx.workspace_bytes(self.M, self.N, self.K)
        self.ws = mx.new_workspace(nws, dev) if nws else None  # zeroed tile counters
        self.mx = mx
        mx.pack_b(self.bq, self.bs, out=self.b_packed)
        torch.cuda.synchronize()

    def pack(self):
        self.mx.pack_b(self.bq, self.bs, out=self.b_packed)

    def call(self):
        self.mx.gemm(self.a, self.b_packed, self.N, out=self.c, workspace=self.ws, plan=self.plan)


def time_cold(torch, flush, fn, steps, warmup):
    """Median/mean µs of fn() with an L2 + Infinity Cache eviction before each call."""
    for _ in range(warmup):
        flush.zero_()
        fn()
    torch.cuda.synchronize()
    evs = []
    for _ in range(steps):
        flush.zero_()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    us = [a.elapsed_time(b) * 1000.0 for a, b in evs]
    return us


def trimmed_mean(us):
    """Mean without the single lowest and highest sample."""
    s = sorted(us)
    return statistics.fmean(s[1:-1]) if len(s) > 2 else statistics.fmean(s)


def kernel_sources_sha():
    """sha256 over the HIP sources; hardware byte counters recorded under
    profiles/ are only reported while the kernels are unchanged."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_scaled_precision_quant_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def recorded_profile(workload):
    """The committed rocprofv3 record for the workload (HBM bytes per launch
    from the FETCH_SIZE/WRITE_SIZE runs, median traced kernel duration), or
    None when the kernel sources have changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("kernel_sources_sha") != kernel_sources_sha():
        return None
    return entry


def cpu_baseline(names, seconds):
    """The oracle as it stands, on the same inputs: quantize A, dequantize A
    and B, fp32 dot.  B's quantization is excluded, as it is in the GPU call
    (B arrives pre-quantized).  Timed on one thread, then on every host core
    the process may use (at most 16): one thread per core, each running
    whole oracle calls (the oracle's C routines release the interpreter
    lock).  About 2*seconds of CPU work in all."""
    import threading

    import oracle
    prepared = []
    for n in names:
        a, b = inputs.make(n)
        bq, bs = oracle.quantize(b)
        prepared.append((a, bq, bs))

    def one_call(a, bq, bs):
        aq, asc = oracle.quantize(a)
        ad = oracle.dequantize(aq, asc)
        bd = oracle.dequantize(bq, bs)
        oracle.gemm(ad, bd, want64=False)

    def run(threads, wall_s):
        counts = [0] * threads
        stop = time.perf_counter() + wall_s

        def worker(i):
            while True:
                for x in prepared:
                    one_call(*x)
                    counts[i] += 1
                if time.perf_counter() >= stop:
                    return
        t0 = time.perf_counter()
        ts = [threading.Thread(target=worker, args=(i,)) for i in range(threads)]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        return time.perf_counter() - t0, sum(counts)

    dt1, n1 = run(1, seconds / 2)
    affinity = len(os.sched_getaffinity(0))
    cores = max(1, min(16, affinity))
    dtn, nn = run(cores, max(1.0, seconds * 1.5 / cores))
    return {"value": dtn / nn * 1e6, "unit": "us/call", "cores": cores, "kind": "oracle",
            "single_thread_value": dt1 / n1 * 1e6,
            "host_cpu_count": os.cpu_count(), "host_affinity": affinity,
            "sample": "full oracle calls over the workload's shapes (%s): %d calls on %d threads "
                      "in %.1f s wall; single thread: %d calls in %.1f s"
                      % (", ".join(names), nn, cores, dtn, n1, dt1)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(one GPU's share of an N-sharded GEMM is the same call); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import block_scaled_precision_quant_amd as mx

    names = WORKLOAD_SETS[args.workload]
    cases = [Case(n, torch, mx) for n in names]
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda:0")
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # timed region: K steps, each one cold call per shape
    for _ in range(args.warmup):
        for c in cases:
            flush.zero_()
            c.call()
    torch.cuda.synchronize()
    ev = {c.name: [] for c in cases}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for c in cases:
            flush.zero_()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            c.call()
            e1.record()
            ev[c.name].append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {}
    for c in cases:
        us = [a.elapsed_time(b) * 1000.0 for a, b in ev[c.name]]
        per[c.name] = {"median_us": statistics.median(us), "mean_us": statistics.fmean(us),
                       "trimmed_mean_us": trimmed_mean(us), "min_us": min(us),
                       "plan": c.plan.__dict__,
                       "alg_bytes": alg_bytes(c.M, c.N, c.K), "flops": 2 * c.M * c.N * c.K}
    value = statistics.fmean(p["median_us"] for p in per.values())

    # the same protocol around the smallest kernel there is (a 1-element
    # fill): the event-timing floor of one launch after the cache eviction
    tiny = torch.zeros(1, dtype=torch.uint8, device="cuda:0")
    floor_us = statistics.median(time_cold(torch, flush, tiny.zero_, 20, 3))

    # dominant kernel: the GEMM kernel; with single-launch plans the event pair
    # brackets exactly that kernel, so achieved = algorithmic bytes per launch
    # over the mean event duration per launch in the timed region
    tot_bytes = sum(p["alg_bytes"] for p in per.values())
    tot_us = sum(p["median_us"] for p in per.values())
    mean_us = statistics.fmean(p["mean_us"] for p in per.values())
    achieved = tot_bytes / len(per) / (mean_us * 1e-6) / 1e9
    tot_flops = sum(p["flops"] for p in per.values())
    prof = recorded_profile(args.workload)
    for c in cases:
        p = per[c.name]
        p["hbm_GBps"] = p["alg_bytes"] / (p["median_us"] * 1e-6) / 1e9
        p["hbm_frac"] = p["hbm_GBps"] / HBM_PEAK_GBPS
        p["mfma_frac"] = p["flops"] / (p["median_us"] * 1e-6) / 1e12 / FP4_PEAK_TFLOPS
        p["prepack_us"] = statistics.median(time_cold(torch, flush, c.pack, 10, 2))

    line = {
        "metric": "L2-cold us/call per (M,N,K) + achieved HBM TB/s and FP4 MFMA % of peak",
        "value": round(value, 3),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4(e2m1)+e8m0 x fp4 -> fp32 acc, bf16 in/out",
        "data": "synthetic (seeded normal A and B, bf16)",
        "config": {"workload": "mxfp4_gemm " + " + ".join(
            "M=%d N=%d K=%d" % (c.M, c.N, c.K) for c in cases), "shapes": per},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": prof and prof.get("bytes_per_launch"),
                     "kernel": "gemm_kernel (one launch per call)",
                     "launch_us_mean": round(mean_us, 3),
                     # the same kernel's rocprofv3 duration (committed trace of this
                     # command): the event pair also brackets dispatch overhead
                     "kernel_us_rocprof": prof and prof.get("kernel_ns_median") and
                     round(prof["kernel_ns_median"] / 1000.0, 3),
                     "achieved_at_kernel_us": prof and prof.get("kernel_ns_median") and
                     round(tot_bytes / len(per) / (prof["kernel_ns_median"] * 1e-9) / 1e9, 1)},
        "event_floor_us": round(floor_us, 3),
        "hbm_TBps": round(achieved / 1000.0, 4),
        "mfma_frac_fp4": round(tot_flops / (tot_us * 1e-6) / 1e12 / FP4_PEAK_TFLOPS, 6),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(names, args.cpu_seconds)
    print(json.dumps(line), flush=True)

    if args.all:
        for n in inputs.ORDER:
            c = Case(n, torch, mx)
            us = time_cold(torch, flush, c.call, args.steps, args.warmup)
            med = statistics.median(us)
            b = alg_bytes(c.M, c.N, c.K)
            alt = {}
            for label, fields in ALTERNATIVES.get(n, {}).items():
                p = mx.Plan(*fields)
                ws = mx.new_workspace(mx.workspace_bytes(c.M, c.N, c.K, p), "cuda:0")
                run = lambda: mx.gemm(c.a, c.b_packed, c.N, out=c.c, workspace=ws, plan=p)
                alt[label] = {"plan": p.__dict__, "median_us": round(statistics.median(
                    time_cold(torch, flush, run, args.steps, args.warmup)), 3)}
            print(json.dumps({"shape": n, "plan": c.plan.__dict__, "median_us": round(med, 3),
                              "mean_us": round(statistics.fmean(us), 3),
                              "trimmed_mean_us": round(trimmed_mean(us), 3),
                              "hbm_GBps": round(b / (med * 1e-6) / 1e9, 1),
                              "mfma_frac_fp4": round(2 * c.M * c.N * c.K / (med * 1e-6) / 1e12
                                                     / FP4_PEAK_TFLOPS, 5),
                              "prepack_us": round(statistics.median(
                                  time_cold(torch, flush, c.pack, 10, 2)), 3),
                              "alternatives": alt}), flush=True)
            del c

    if args.large:
        for i, (M, N, K) in enumerate(LARGE):
            w = inputs.Workload("large_m%d_n%d_k%d" % (M, N, K), M, N, K, seed=100 + i)
            c = Case(w, torch, mx)
            steps = max(3, min(args.steps, 20))
            us = time_cold(torch, flush, c.call, steps, 2)
            ap = mx.quant_a_packed(c.a)
            pre = lambda: mx.gemm_prequant(ap, M, c.b_packed, N, K, out=c.c, plan=c.plan)
            us_pre = time_cold(torch, flush, pre, steps, 2)
            fl = 2.0 * M * N * K
            med, med_pre = statistics.median(us), statistics.median(us_pre)
            print(json.dumps({"shape": w.name, "plan": c.plan.__dict__, "median_us": round(med, 3),
                              "mfma_frac_fp4": round(fl / (med * 1e-6) / 1e12 / FP4_PEAK_TFLOPS, 4),
                              "prequant_A_median_us": round(med_pre, 3),
                              "prequant_A_mfma_frac_fp4": round(
                                  fl / (med_pre * 1e-6) / 1e12 / FP4_PEAK_TFLOPS, 4),
                              "hbm_GBps": round(alg_bytes(M, N, K) / (med * 1e-6) / 1e9, 1)}),
                  flush=True)
            del c, ap
            torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
