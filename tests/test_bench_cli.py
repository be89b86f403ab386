"""bench.py's command line on the host: more than one GPU is refused with a message
(the R ranks are partitions of one GPU), before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, env=env)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_a_multi_rank_launch_is_refused():
    env = dict(os.environ, WORLD_SIZE="8")
    r = _run(env=env)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
