"""bench.py's host-side contract: a launch on more than one GPU is refused before any device
work, with a message and exit status 2 and no JSON line."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT, env=env)


def test_bench_refuses_more_than_one_gpu():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_bench_refuses_a_multi_rank_launch():
    r = _run([], env=dict(os.environ, WORLD_SIZE="2", RANK="0", LOCAL_RANK="0"))
    assert r.returncode == 2
    assert "WORLD_SIZE 2" in r.stderr
    assert r.stdout == ""
