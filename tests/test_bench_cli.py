"""bench.py's command line on the host: more than one GPU is refused with a
message before any device work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_cpu_baseline_is_one_full_oracle_call_at_the_headline_workload():
    import importlib.util

    import workloads as wk

    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    assert bench.cpu_tokens(wk.WORKLOADS[3], 0) == 8192  # 25.8 TFLOP: the whole workload
    assert bench.cpu_tokens(wk.WORKLOADS[2], 0) == 4096
    n5 = bench.cpu_tokens(wk.WORKLOADS[5], 0)  # 116 TFLOP: the first whole tiles within budget
    assert n5 % 256 == 0 and 0 < n5 < 32768
    assert 6.0 * n5 * 256000 * 2304 <= bench.CPU_BUDGET_FLOPS
    assert bench.cpu_tokens(wk.WORKLOADS[3], 1000) == 1000
