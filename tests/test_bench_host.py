"""Host-side checks of bench.py (no GPU needed): the oracle-only timing mode and
the refusal of runs over several GPUs."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def run_bench(*args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, env=env, timeout=300)


def test_cpu_only_ring_run_reports_the_threads_it_used():
    r = run_bench("--workload", "1", "--cpu-only", "--cpu-seconds", "0.2", env_extra={"OMP_NUM_THREADS": "2"})
    assert r.returncode == 0, r.stderr
    line = json.loads(r.stdout.strip().splitlines()[-1])
    cb = line["cpu_baseline"]
    assert line["workload"] == 1
    assert cb["kind"] == "oracle" and cb["unit"] == "query-heads/s"
    assert cb["cores"] == 2  # the count the oracle's loops were set to, read back
    assert cb["value"] > 0


def test_cpu_only_decode_sample():
    r = run_bench("--workload", "2", "--cpu-only", "--cpu-seconds", "0.5", env_extra={"OMP_NUM_THREADS": "1"})
    assert r.returncode == 0, r.stderr
    cb = json.loads(r.stdout.strip().splitlines()[-1])["cpu_baseline"]
    assert cb["cores"] == 1 and cb["value"] > 0
    assert "queries" in cb["sample"]


def test_several_gpus_are_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_tiny_ring_run_is_not_a_gpu_bench_line():
    r = run_bench("--workload", "1")
    assert r.returncode == 2
    assert "--cpu-only" in r.stderr
