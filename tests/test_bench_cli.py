"""bench.py runs on one GPU only: asked for more (by flag or by a launcher's
WORLD_SIZE) it exits with status 2 and says why, before touching a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, env=env, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "single-GPU" in r.stderr and r.stdout == ""


def test_launcher_world_size_is_refused():
    r = _bench(["--gpus", "1"], {"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "WORLD_SIZE 4" in r.stderr
