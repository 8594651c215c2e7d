"""Host-side logic of bench.py (CPU only): the algorithmic byte count per
call, the trimmed mean, the one-GPU guard, and the plan alternatives it
times."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_alg_bytes_match_the_config_sizes():
    # A bf16 + B fp4 + B e8m0 + C bf16, e.g. M=4 N=2880 K=512:
    # 4,096 + 737,280 + 46,080 + 23,040
    assert bench.alg_bytes(4, 2880, 512) == 810496
    assert bench.alg_bytes(32, 4096, 512) == 1409024
    assert bench.alg_bytes(16, 2112, 7168) == 229376 + 7569408 + 473088 + 67584
    assert bench.alg_bytes(256, 3072, 1536) == 786432 + 2359296 + 147456 + 1572864


def test_trimmed_mean_drops_one_low_and_one_high():
    assert bench.trimmed_mean([1.0, 2.0, 3.0, 100.0]) == 2.5
    assert bench.trimmed_mean([5.0, 7.0]) == 6.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_alternative_plans_are_valid():
    mx = pytest.importorskip("block_scaled_precision_quant_amd")
    try:
        mx.load()
    except (ImportError, OSError) as e:
        pytest.skip("library not built: %s" % e)
    from block_scaled_precision_quant_amd import inputs
    for name, alts in bench.ALTERNATIVES.items():
        w = inputs.WORKLOADS[name]
        for fields in alts.values():
            mx.check_plan(mx.Plan(*fields), w.M, w.N, w.K)
    for M, N, K in bench.LARGE + bench.STREAM:  # the extra lines' default plans
        mx.check_plan(mx.default_plan(M, N, K), M, N, K)


def test_recorded_profile_matches_the_kernel_sources():
    """profiles/traffic.json (the rocprofv3 record bench.py reads for kernel
    durations, HBM bytes and counters) was taken with the current kernel
    sources and covers every benchmark shape with the plan its default still
    is; a kernel change, or a plan-rule change that moves a benchmark shape,
    without a new profile fails here, before a bench line reports stale
    figures."""
    from block_scaled_precision_quant_amd import inputs
    rec = bench.recorded_profiles()
    assert rec, "profiles/traffic.json is missing or was taken with other kernel sources"
    assert set(rec["shapes"]) == set(inputs.ORDER)
    for name, e in rec["shapes"].items():
        w = inputs.WORKLOADS[name]
        assert e["alg_bytes"] == bench.alg_bytes(w.M, w.N, w.K)
        assert e["kernel_us"] > 0 and e["hbm_bytes_per_call"] > 0
    assert rec["empty_kernel_us"]["median"] > 0
