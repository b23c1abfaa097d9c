"""Host checks of bench.py's command line (no GPU): it measures one GPU and
says so for any other count, and rejects option combinations it does not run,
before it touches the GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("n", ["2", "8", "0"])
def test_other_gpu_counts_exit_with_a_message(n):
    r = _bench("--gpus", n)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""          # no JSON line for a run that did not happen


def test_reuse_every_must_be_positive():
    r = _bench("--reuse-every", "0")
    assert r.returncode != 0 and "--reuse-every must be >= 1" in r.stderr
