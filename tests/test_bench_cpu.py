"""Host-side checks of bench.py's command line: it measures one GPU and says
so when asked for more (no GPU is needed for these)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_a_multi_rank_launch_is_refused_with_a_message():
    r = _bench([], env=dict(os.environ, WORLD_SIZE="4"))
    assert r.returncode == 2
    assert "one GPU" in r.stderr
