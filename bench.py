"""Benchmark: L2-cold microseconds per MXFP4 GEMM call on one MI355X, for each
of the six benchmark shapes of the amd-mxfp4-mm pages.

One step is one call of every shape (4x2880x512, 32x4096x512, 32x2880x512,
16x2112x7168, 64x7168x2048, 256x3072x1536).  Before every timed call a
512 MiB device fill evicts the L2 caches and the Infinity Cache, and HIP
events on the launch stream bracket the call alone (launch and scheduling
included).  The kernels' own durations come from rocprofv3 traces of this
same command, recorded under profiles/ with the kernel sources' sha256 and
used only while the sources still match.
Inputs (A bf16, packed B) are resident in HBM before timing starts; B is
quantized by the library's quantizer and repacked once (timed separately,
prepack_us).

Prints one JSON line.  `value` is the median L2-cold event time per call of
the largest shape by bytes, 64x7168x2048 (us, lower is better); every shape's
figures are under config.shapes.  `roofline` is that shape's GEMM kernel
against the HBM peak: algorithmic bytes over the kernel's traced duration
(`frac`), and over the live event time per call (`frac_event`); `fp4_mfma`
is the compute-leaning 256x3072x1536 shape against the dense FP4 peak.
`ms_per_step` is wall time per step, cache-evicting fills included.

  python bench.py [--steps K] [--warmup W] [--alternatives] [--large] [--stream]
                  [--no-cpu-baseline] [--cpu-seconds S] [--copy-calibration]

--alternatives adds one line per shape that has a choice, timing the other
plans (A pre-quantized by a separate launch, the tiled kernel) the same way.
--large adds one line per large shape (M >= 1024), whose default plan is the
tiled kernel.  --stream adds one line per weight-streaming shape (small M, a
B of 60-150 MB), timed through the default plan the same way.
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
VALUE_SHAPE = "m64_n7168_k2048"    # the largest shape by bytes: headline value and HBM roofline
MFMA_SHAPE = "m256_n3072_k1536"    # the compute-leaning shape: FP4 matrix-core fraction

# The pages' own figures for this path, quoted as context only (another
# harness on the same GPU model; not a target): submission 705642's notes on
# the library baseline at M=4.
PAGES_CONTEXT = {
    "library_baseline_us_m4": 8.2,
    "memory_floor_us_m4": 0.13,
    "source": "kernelindex.com kernelbot-amd-mxfp4-mm-705642, v3 docstring (anatomy of the "
              "library baseline at M=4): about 8.2 us per call against a memory floor of "
              "about 0.13 us; context only",
    "hip_fused_quant_split_k_us_m64": 10.0,
    "source_m64": "kernelindex.com kernelbot-amd-mxfp4-mm-739530, v5 HIP source, the comment "
                  "heading the fused-quant split-K kernel (fgemm_fq): about 10.0 us per call at "
                  "m=64, shape not stated (the pages' one m=64 benchmark shape is "
                  "64x7168x2048); context only",
}


def alg_bytes(M, N, K):
    """Bytes the method itself must move per call: A bf16, B fp4 + e8m0, C bf16."""
    return 2 * M * K + N * K // 2 + N * K // 32 + 2 * M * N


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--alternatives", action="store_true",
                    help="one extra JSON line per shape with a plan choice")
    ap.add_argument("--large", action="store_true",
                    help="one extra JSON line per large shape (tiled kernel)")
    ap.add_argument("--stream", action="store_true",
                    help="one extra JSON line per weight-streaming shape (small M, large N x K)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=3.0,
                    help="wall seconds of the all-cores oracle run (plus one single-thread "
                         "call per shape)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 64 MiB device copy first (a known-size kernel for "
                         "scaling hardware byte counters)")
    return ap.parse_args(argv)


# large shapes for --large: (M, N, K), seeded like the workloads; the last has
# few tiles and a long K (the tiled mode splits K over workgroups)
LARGE = [(1024, 8192, 8192), (4096, 4096, 4096), (8192, 8192, 8192), (256, 8192, 28672)]
# weight-streaming shapes for --stream: (M, N, K), B of 60-150 MB
STREAM = [(1, 16384, 16384), (16, 16384, 16384), (64, 16384, 16384), (32, 28672, 8192),
          (16, 8192, 28672)]

# --alternatives: the other plans where a shape makes a choice -- the fastest
# pre-quantized-A plan of an L2-cold sweep over every valid plan (a separate
# quantizer launch, then the GEMM) and the tiled mode.  Fields: mode,
# m_blocks, n_tiles_per_wave, waves_n, waves_k, k_steps_per_wave, split_k.
ALTERNATIVES = {
    "m64_n7168_k2048": {"prequant": (2, 2, 1, 4, 2, 8, 1)},
    "m256_n3072_k1536": {"prequant": (2, 2, 1, 6, 1, 12, 1), "tiled": (3, 1, 1, 2, 1, 1, 1)},
}


class Case:
    """Device-resident inputs and outputs of one shape."""

    def __init__(self, name, torch, mx, plan=None):
        w = inputs.WORKLOADS[name] if isinstance(name, str) else name
        self.name, self.M, self.N, self.K = w.name, w.M, w.N, w.K
        a_bits, b_bits = inputs.make(w)
        dev = torch.device("cuda:0")
        to = lambda bits: torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
        self.a = to(a_bits)
        b = to(b_bits)
        self.bq, self.bs = mx.quant_a(b)  # the library's quantizer on B's rows
        self.b_packed = torch.empty(mx.packed_bytes(self.N, self.K), dtype=torch.uint8, device=dev)
        self.c = torch.empty((self.M, self.N), dtype=torch.bfloat16, device=dev)
        self.plan = plan or mx.default_plan(self.M, self.N, self.K)
        nws = mx.workspace_bytes(self.M, self.N, self.K, self.plan)
        self.ws = mx.new_workspace(nws, dev) if nws else None  # zeroed tile counters
        self.mx = mx
        mx.pack_b(self.bq, self.bs, out=self.b_packed)
        torch.cuda.synchronize()

    def pack(self):
        self.mx.pack_b(self.bq, self.bs, out=self.b_packed)

    def call(self):
        self.mx.gemm(self.a, self.b_packed, self.N, out=self.c, workspace=self.ws, plan=self.plan)

    def launches(self):
        # the GEMM kernel, the quantizer of A (pre-quantized, tiled, stream),
        # the reduce kernel (split plans that use it; tiled and stream ones always)
        p = self.plan
        return 1 + (p.mode in (2, 3, 4)) + (p.split_k > 1 and (p.mode in (3, 4) or p.split_reduce == 0))


def time_cold(torch, flush, cases, steps, warmup):
    """Per case: event microseconds of `steps` calls, each after a
    cache-evicting fill.  Returns ({name: [us]}, wall seconds of the timed
    steps)."""
    for _ in range(warmup):
        for c in cases:
            flush.zero_()
            c.call()
    torch.cuda.synchronize()
    evs = {c.name: [] for c in cases}
    t0 = time.perf_counter()
    for _ in range(steps):
        for c in cases:
            flush.zero_()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            c.call()
            e1.record()
            evs[c.name].append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return {n: [a.elapsed_time(b) * 1e3 for a, b in v] for n, v in evs.items()}, wall


def time_cold_fn(torch, flush, fn, steps, warmup):
    """Event microseconds of fn() after a cache-evicting fill (for calls that
    are not workload calls: the pre-pack, the 1-byte fill)."""
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
    return [a.elapsed_time(b) * 1000.0 for a, b in evs]


def trimmed_mean(us):
    """Mean without the single lowest and highest sample."""
    s = sorted(us)
    return statistics.fmean(s[1:-1]) if len(s) > 2 else statistics.fmean(s)


def kernel_sources_sha():
    """sha256 over the device sources (the .hip files and the headers they
    share); hardware counters recorded under profiles/ are only reported
    while the kernels are unchanged.  The host-side plan choice (api.cpp) is
    checked per shape instead: see recorded_profiles."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_scaled_precision_quant_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if not f.endswith((".hip", ".hpp")):
            continue
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def recorded_profiles():
    """The committed rocprofv3 record of this command (profiles/traffic.json:
    per shape the traced kernel durations, HBM bytes per call from the
    FETCH_SIZE/WRITE_SIZE runs and, for the compute-leaning shape, matrix-core
    counters; the empty-kernel durations of the same trace), only while the
    kernel sources hash to the sha it was taken with ({} otherwise), and of
    those shapes only the ones whose default plan is still the plan recorded
    with them."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return {}
    if rec.get("kernel_sources_sha") != kernel_sources_sha():
        return {}
    import block_scaled_precision_quant_amd as mx
    keep = {}
    for name, e in rec.get("shapes", {}).items():
        w = inputs.WORKLOADS.get(name)
        if w is not None and e.get("plan") == mx.default_plan(w.M, w.N, w.K).__dict__:
            keep[name] = e
    return dict(rec, shapes=keep)


def shape_label(c):
    return "M=%d N=%d K=%d" % (c.M, c.N, c.K)


def summarize(c, ev, prof):
    b, fl = alg_bytes(c.M, c.N, c.K), 2 * c.M * c.N * c.K
    med = statistics.median(ev)
    out = {
        "median_us": round(med, 3), "trimmed_mean_us": round(trimmed_mean(ev), 3),
        "mean_us": round(statistics.fmean(ev), 3), "min_us": round(min(ev), 3),
        "launches": c.launches(), "plan": c.plan.__dict__, "alg_bytes": b, "flops": fl,
        "hbm_frac_event": round(b / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "mfma_frac_event": round(fl / (med * 1e-6) / 1e12 / FP4_PEAK_TFLOPS, 5),
    }
    p = prof.get(c.name)
    if p:
        k = p["kernel_us"]  # sum of the call's kernels' median traced durations
        out["kernel_us"] = k
        out["kernels"] = p.get("kernels")
        out["hbm_frac_kernel"] = round(b / (k * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
        out["mfma_frac_kernel"] = round(fl / (k * 1e-6) / 1e12 / FP4_PEAK_TFLOPS, 5)
        if p.get("hbm_bytes_per_call"):
            out["hbm_bytes_counted"] = p["hbm_bytes_per_call"]
            out["hbm_bytes_over_alg"] = round(p["hbm_bytes_per_call"] / b, 3)
    return out


def cpu_baseline(names, main_name, seconds):
    """The oracle as it stands, on the same inputs: quantize A, dequantize A
    and B, fp32 dot.  B's quantization is excluded, as it is in the GPU call
    (B arrives pre-quantized).  One call of every shape on one thread, then
    whole calls of the main shape on every host core the process may use (at
    most 16, one thread each; the oracle's C routines release the
    interpreter lock) for about `seconds` of wall time."""
    import threading

    import oracle
    prepared = {}
    for n in names:
        a, b = inputs.make(n)
        bq, bs = oracle.quantize(b)
        prepared[n] = (a, bq, bs)

    def one_call(a, bq, bs):
        aq, asc = oracle.quantize(a)
        ad = oracle.dequantize(aq, asc)
        bd = oracle.dequantize(bq, bs)
        oracle.gemm(ad, bd, want64=False)

    single = {}
    for n in names:
        t0 = time.perf_counter()
        one_call(*prepared[n])
        single[n] = round((time.perf_counter() - t0) * 1e6, 1)

    affinity = len(os.sched_getaffinity(0))
    cores = max(1, min(16, affinity))
    counts = [0] * cores
    stop = time.perf_counter() + seconds

    def worker(i):
        while True:
            one_call(*prepared[main_name])
            counts[i] += 1
            if time.perf_counter() >= stop:
                return
    t0 = time.perf_counter()
    ts = [threading.Thread(target=worker, args=(i,)) for i in range(cores)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    wall = time.perf_counter() - t0
    calls = sum(counts)
    return {"value": round(wall / calls * 1e6, 1), "unit": "us/call", "cores": cores,
            "kind": "oracle", "shape": main_name,
            "single_thread_us_per_call": single,
            "host_cpu_count": os.cpu_count(), "host_affinity": affinity,
            "sample": "%d whole oracle calls of %s on %d threads in %.1f s wall (value = wall / "
                      "calls); one call of each shape on one thread (single_thread_us_per_call)"
                      % (calls, main_name, cores, wall)}


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(one GPU's share of an N-sharded GEMM is the same call); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import block_scaled_precision_quant_amd as mx

    cases = [Case(n, torch, mx) for n in inputs.ORDER]
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda:0")
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ev, wall = time_cold(torch, flush, cases, args.steps, args.warmup)
    rec = recorded_profiles()
    prof = rec.get("shapes", {})
    per = {c.name: summarize(c, ev[c.name], prof) for c in cases}
    for c in cases:
        pp = statistics.median(time_cold_fn(torch, flush, c.pack, 10, 2))
        per[c.name]["prepack_us"] = round(pp, 3)
        # the one-time repack reads and writes N*K/2 + N*K/32 bytes
        per[c.name]["prepack_GBps_event"] = round(2 * (c.N * c.K // 2 + c.N * c.K // 32)
                                                  / (pp * 1e-6) / 1e9, 1)

    # the same protocol around the smallest kernel there is (a 1-element
    # fill): the event-time floor of one launch after the cache eviction
    tiny = torch.zeros(1, dtype=torch.uint8, device="cuda:0")
    floor = time_cold_fn(torch, flush, tiny.zero_, 20, 3)

    main_case = next(c for c in cases if c.name == VALUE_SHAPE)
    mfma_case = next(c for c in cases if c.name == MFMA_SHAPE)
    vb = alg_bytes(main_case.M, main_case.N, main_case.K)
    e_mean = statistics.fmean(ev[VALUE_SHAPE])
    mp = prof.get(VALUE_SHAPE, {})
    main_kernel = (mp.get("kernels") or [{}])[0]
    if main_kernel.get("mean_us"):
        # the GEMM kernel's average traced duration in this same command
        k_mean = main_kernel["mean_us"]
        basis = "rocprofv3 kernel trace of this command (profiles/), average duration"
    else:
        k_mean = e_mean
        basis = "event time per call (no kernel trace recorded for these kernel sources)"
    achieved = vb / (k_mean * 1e-6) / 1e9
    mfl = 2 * mfma_case.M * mfma_case.N * mfma_case.K
    mprof = prof.get(MFMA_SHAPE, {})
    m_us = mprof.get("kernel_us")

    line = {
        "metric": "L2-cold us/call per (M,N,K) + achieved HBM TB/s and FP4 MFMA % of peak",
        "value": per[VALUE_SHAPE]["median_us"],
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
        "config": {
            "workload": "mxfp4_gemm, the six benchmark shapes: " + "; ".join(
                shape_label(c) for c in cases),
            "value_shape": shape_label(main_case),
            "shapes": per,
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": mp.get("hbm_bytes_per_call"),
            "kernel": (main_kernel.get("name") or "gemm_kernel") + " at " + shape_label(main_case),
            "kernel_us_mean": round(k_mean, 3), "basis": basis,
            "event_us_mean": round(e_mean, 3),
            "achieved_event": round(vb / (e_mean * 1e-6) / 1e9, 1),
            "frac_event": round(vb / (e_mean * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        },
        "fp4_mfma": {
            "shape": shape_label(mfma_case), "peak_tflops": FP4_PEAK_TFLOPS,
            "frac_kernel": m_us and round(mfl / (m_us * 1e-6) / 1e12 / FP4_PEAK_TFLOPS, 5),
            "frac_event": per[MFMA_SHAPE]["mfma_frac_event"],
            "counters": mprof.get("mfma_counters"),
        },
        "event_floor_us": {"median": round(statistics.median(floor), 3),
                           "min": round(min(floor), 3)},
        "empty_kernel_us_rocprof": rec.get("empty_kernel_us"),
        "pages_context": PAGES_CONTEXT,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inputs.ORDER, VALUE_SHAPE, args.cpu_seconds)
    print(json.dumps(line), flush=True)

    if args.alternatives:
        for n, alts in ALTERNATIVES.items():
            base = next(c for c in cases if c.name == n)
            out = {"shape": n, "default": {"plan": base.plan.__dict__,
                                           "median_us": per[n]["median_us"]}}
            for label, fields in alts.items():
                c = Case(n, torch, mx, plan=mx.Plan(*fields))
                e, _ = time_cold(torch, flush, [c], args.steps, args.warmup)
                out[label] = {"plan": c.plan.__dict__,
                              "median_us": round(statistics.median(e[n]), 3)}
                del c
            print(json.dumps(out), flush=True)

    if args.large:
        for i, (M, N, K) in enumerate(LARGE):
            w = inputs.Workload("large_m%d_n%d_k%d" % (M, N, K), M, N, K, seed=100 + i)
            c = Case(w, torch, mx)
            steps = max(3, min(args.steps, 20))
            e, _ = time_cold(torch, flush, [c], steps, 2)
            ap = mx.quant_a_packed(c.a)
            nws = mx.prequant_workspace_bytes(M, N, K, c.plan)  # split partials, allocated once
            ws_pre = mx.new_workspace(nws, c.a.device) if nws else None
            pre = lambda: mx.gemm_prequant(ap, M, c.b_packed, N, K, out=c.c, workspace=ws_pre, plan=c.plan)
            us_pre = time_cold_fn(torch, flush, pre, steps, 2)
            fl = 2.0 * M * N * K
            med, med_pre = statistics.median(e[w.name]), statistics.median(us_pre)
            print(json.dumps({"shape": w.name, "plan": c.plan.__dict__, "median_us": round(med, 3),
                              "mfma_frac_event": round(fl / (med * 1e-6) / 1e12 / FP4_PEAK_TFLOPS, 4),
                              "prequant_A_median_us": round(med_pre, 3),
                              "prequant_A_mfma_frac_event": round(
                                  fl / (med_pre * 1e-6) / 1e12 / FP4_PEAK_TFLOPS, 4)}),
                  flush=True)
            del c, ap, ws_pre
            torch.cuda.empty_cache()

    if args.stream:
        dev = torch.device("cuda:0")
        for i, (M, N, K) in enumerate(STREAM):
            # seeded normal inputs drawn on the device (B alone is up to 512 MiB of bf16)
            gen = torch.Generator(device=dev).manual_seed(200 + i)
            a = torch.randn((M, K), dtype=torch.bfloat16, device=dev, generator=gen)
            b = torch.randn((N, K), dtype=torch.bfloat16, device=dev, generator=gen)
            bq, bs = mx.quant_a(b)
            del b
            bp = mx.pack_b(bq, bs)
            del bq, bs
            c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            plan = mx.default_plan(M, N, K)
            nws = mx.workspace_bytes(M, N, K, plan)
            ws = mx.new_workspace(nws, dev) if nws else None
            us = time_cold_fn(torch, flush, lambda: mx.gemm(a, bp, N, out=c, workspace=ws, plan=plan),
                              max(3, min(args.steps, 20)), 2)
            med = statistics.median(us)
            ab = alg_bytes(M, N, K)
            print(json.dumps({"shape": "stream_m%d_n%d_k%d" % (M, N, K), "plan": plan.__dict__,
                              "median_us": round(med, 3), "alg_bytes": ab,
                              "alg_TBps_event": round(ab / med / 1e6, 3),
                              "hbm_frac_event": round(ab / med / 1e3 / HBM_PEAK_GBPS, 4)}),
                  flush=True)
            del a, bp, c, ws
            torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
