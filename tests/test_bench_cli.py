"""bench.py's host-side contract that needs no GPU: one GPU only."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          env=env, capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    p = run(["--gpus", "2"])
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def test_world_size_above_one_is_refused():
    p = run(["--gpus", "1"], {"WORLD_SIZE": "4"})
    assert p.returncode == 2
    assert "one GPU" in p.stderr
