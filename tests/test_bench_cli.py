"""bench.py's command line on the host (no GPU needed): it measures one GPU and
refuses, with a message, any request for more."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    for argv in (["--gpus", "2"], ["--gpus", "8"]):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode != 0
        assert "one GPU" in r.stderr


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True,
                       text=True, timeout=120, env=env)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
