"""bench.py measures one GPU: asked for more, it exits with a message (CPU)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, env=e, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr
    assert r.stdout.strip() == ""


def test_distributed_launch_is_refused():
    r = _run([], env={"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert r.stdout.strip() == ""
