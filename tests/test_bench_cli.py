"""bench.py's command line on the CPU: it measures one GPU only and says so."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_traffic_reported_only_for_the_profiled_kernel_source(monkeypatch):
    """roofline.traffic comes from the committed counter summary only while the
    kernel sources hash to the value recorded with the counters; after any
    change to them it is null until the counters are taken again."""
    import json
    bench = _bench_module()
    with open(bench.PMC_FILE) as f:
        line = next(l for l in f if l.startswith("pmc: "))
    d = json.loads(line[5:])
    # the summary itself: each K/V byte read about once
    assert 1.0 <= d["traffic_bytes_per_launch"] / d["algorithmic_bytes_per_launch"] < 1.05
    monkeypatch.setattr(bench, "kernel_hash", lambda sources=None: d["kernel_hash"])
    assert bench.traffic_from_profiles() == d["traffic_bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_hash", lambda sources=None: "0" * 16)
    assert bench.traffic_from_profiles() is None


def test_cpu_baseline_uses_every_host_core_and_reports_each_workload():
    """The CPU baseline runs the oracle with BLAS on all the cores the process
    may use, names the CPU, and gives a figure per workload (median of three
    samples for the tiny and the headline workload)."""
    import workloads as wl
    bench = _bench_module()
    cores = bench.host_cores()
    assert 1 <= cores <= len(os.sched_getaffinity(0))
    tiny = wl.CONFIGS["tiny"]
    small = wl.GQAConfig("small", 30, 3, 8, 2, 64, 16, wl.BF16, wl.BF16, "uniform:16:200")
    cases = {"tiny": (tiny, wl.make_gqa_case(tiny)), "small": (small, wl.make_gqa_case(small))}
    r = bench.cpu_baseline(cases, "small", 0.6)
    assert r["cores"] == cores and r["kind"] == "oracle"
    assert set(r["per_config"]) == {"tiny", "small"}
    assert r["per_config"]["tiny"]["samples"] == 3 and r["per_config"]["small"]["samples"] == 3
    assert r["value"] == r["per_config"]["small"]["value"] > 0
    lo, hi = r["per_config"]["small"]["spread_GBps"]
    assert lo <= r["value"] <= hi


def test_mla_counters_reported_only_for_the_profiled_kernel_source(monkeypatch):
    """The MLA roofline block carries traffic and SQ-counter fractions from the
    committed summaries only while the MLA kernel sources hash to the value
    recorded with them."""
    import json
    bench = _bench_module()
    sq = os.path.join(bench.ROOT, "profiles", "mla_sq_counters.md")
    rec = json.loads(next(l for l in open(sq) if l.startswith("sq: "))[4:])
    pmc = json.loads(next(l for l in open(bench.MLA_PMC_FILE) if l.startswith("pmc: "))[5:])
    monkeypatch.setattr(bench, "kernel_hash", lambda sources=None: rec["kernel_hash"])
    d = bench.counters_from_profiles(sq, bench.MLA_KERNEL_SOURCES)
    assert d is not None and 0.0 < d["mfma_busy_frac"] < 1.0
    monkeypatch.setattr(bench, "kernel_hash", lambda sources=None: pmc["kernel_hash"])
    assert bench.traffic_from_profiles(bench.MLA_PMC_FILE, bench.MLA_KERNEL_SOURCES) == pmc["traffic_bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_hash", lambda sources=None: "0" * 16)
    assert bench.counters_from_profiles(sq, bench.MLA_KERNEL_SOURCES) is None
    assert bench.traffic_from_profiles(bench.MLA_PMC_FILE, bench.MLA_KERNEL_SOURCES) is None


def test_headline_kernel_names_each_workloads_own_kernel():
    """The headline roofline names the kernel the library runs for the chosen
    workload and reads HBM counters only from the summary of that workload."""
    import dataclasses
    import workloads as wl
    bench = _bench_module()
    c = wl.CONFIGS
    assert bench.headline_kernel(c["llama8b"], 1, True) == ("gqa_mfma_kernel", bench.KERNEL_SOURCES, bench.PMC_FILE)
    # another GQA workload on the same kernel: no borrowed counters
    assert bench.headline_kernel(c["skewed"], 1, True) == ("gqa_mfma_kernel", bench.KERNEL_SOURCES, None)
    assert bench.headline_kernel(c["llama8b"], 2, True)[2] is None
    assert bench.headline_kernel(c["llama8b"], 1, False)[2] is None
    # fp8 caches run on the matrix-core kernel at every group size
    fp8_small_group = dataclasses.replace(c["longfp8"], q_heads=2 * c["longfp8"].kv_heads)
    assert bench.headline_kernel(fp8_small_group, 1, True)[0] == "gqa_mfma_kernel"
    assert bench.headline_kernel(c["mla"], 1, True) == ("mla_wave_kernel", bench.MLA_KERNEL_SOURCES, bench.MLA_PMC_FILE)
    assert bench.headline_kernel(dataclasses.replace(c["mla"], q_heads=16), 1, False) == ("mla_attn_kernel", None, None)
    assert bench.headline_kernel(c["tiny"], 1, True)[2] is None
