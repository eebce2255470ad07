"""Host-side contract of bench.py (no GPU): it measures one GPU only."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT,
                          env=env, capture_output=True, text=True, timeout=120)


def test_bench_refuses_several_gpus():
    r = run_bench(["--gpus", "2"])
    assert r.returncode == 2, r.stderr
    assert "one GPU" in r.stderr and r.stdout == ""


def test_bench_refuses_a_distributed_launch():
    r = run_bench([], {"WORLD_SIZE": "2"})
    assert r.returncode == 2, r.stderr
    assert "one GPU" in r.stderr and r.stdout == ""
