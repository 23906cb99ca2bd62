"""bench.py's command line on the CPU: more than one GPU is refused with a
message before anything touches a device, and the workload's step count
bounds warm-up + timed steps."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU only" in msg["error"]


def test_steps_beyond_the_workload_are_refused():
    r = _run("--steps", "100", "--warmup", "5")
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "exceeds the workload's" in msg["error"]
