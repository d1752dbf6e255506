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
    monkeypatch.setattr(bench, "kernel_hash", lambda: d["kernel_hash"])
    assert bench.traffic_from_profiles() == d["traffic_bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0" * 16)
    assert bench.traffic_from_profiles() is None
