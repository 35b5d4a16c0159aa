"""bench.py's one-GPU contract, checked without a GPU: a request for several GPUs (by flag or by
a launcher's WORLD_SIZE) ends with a message and exit status 2 before anything is measured."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], env=env,
                          capture_output=True, text=True, timeout=120)


def test_several_gpus_by_flag_are_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_several_ranks_by_launcher_are_refused():
    r = _run(["--gpus", "1"], {"WORLD_SIZE": "8"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr
