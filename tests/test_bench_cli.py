"""bench.py's command line on the CPU: the one-GPU guard and argument checks
run before anything touches a GPU."""
import os
import subprocess
import sys

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=REPO)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(REPO, "bench.py")], capture_output=True,
                       text=True, timeout=120, cwd=REPO, env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_zero_streams_is_an_argument_error():
    r = _run("--streams", "0")
    assert r.returncode == 2
    assert "--streams must be at least 1" in r.stderr
