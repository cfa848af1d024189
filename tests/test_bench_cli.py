"""bench.py's command line on the CPU: a request for more than one GPU exits
with status 2 and says why, before touching any device; the measurement modes
are all listed."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_modes_listed():
    r = _run("--help")
    assert r.returncode == 0
    for mode in ("fwd", "gdn", "decode", "bwd", "varlen", "bwd_varlen", "mixer", "strong"):
        assert mode in r.stdout
