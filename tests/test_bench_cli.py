"""bench.py's command line on the host (no GPU): the one-GPU contract and the
presets of the five stream configurations."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _args(*argv):
    old = sys.argv
    sys.argv = ["bench.py", *argv]
    try:
        return bench.parse()
    finally:
        sys.argv = old


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_presets_are_the_five_configurations():
    assert bench.default_workload(_args())
    assert bench.config_workload(_args()) == 3
    for n in (1, 2, 3, 4, 5):
        a = _args("--config", str(n))
        assert bench.config_workload(a) == n
        assert bench.default_workload(a) == (n == 3)
    a = _args("--config", "1")
    assert (a.layers, a.heads, a.image_tokens, a.window, a.frames, a.dtype) == (1, 2, 32, 4, 64, "fp32")
    a = _args("--config", "2")
    assert (a.layers, a.window, a.key_offset_std) == (1, 16, 0.5)
    a = _args("--config", "4")
    assert (a.window, a.frames) == (2000, 2000)
    a = _args("--config", "5")
    assert (a.image_tokens, a.reset_every) == (999, 128)
    # a variant is not a configuration line
    assert bench.config_workload(_args("--rotary")) == 0
    assert not bench.default_workload(_args("--summary-tokens", "1"))
