"""bench.py's command-line contract that holds without a GPU: a run on more than
one GPU (or under a multi-rank launcher) is refused with a message and a non-zero
exit status before anything touches a device, because the library has no
multi-GPU path to time."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, env=e, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_multi_rank_launch_is_refused():
    r = _bench([], env={"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "WORLD_SIZE=4" in r.stderr
