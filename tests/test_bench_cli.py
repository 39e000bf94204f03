"""bench.py's command line, without a device: more than one GPU is refused
with a message, and the help lists every mode."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    res = _run("--gpus", "2", "--no-cpu-baseline")
    assert res.returncode != 0
    assert "one GPU" in (res.stdout + res.stderr)


def test_help_lists_the_modes():
    res = _run("--help")
    assert res.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--workload", "--path", "--form",
                 "--sinkhorn-sweep", "--n-sweep", "--backward", "--all-configs", "--crossover",
                 "--cooperative"):
        assert flag in res.stdout, flag
