"""bench.py's command line on the host: more than one GPU is refused with a message, before any
GPU work (the fit and fill run on a single GPU)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT, env=env)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = _run("--gpus", n)
        assert r.returncode == 2, r.stderr
        assert "one GPU" in r.stderr and not r.stdout


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = _run(env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr
