"""bench.py's command line on a host without a GPU: it measures one GPU only,
so any other --gpus value ends at once with a message and status 2, before
anything touches a device."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", ["2", "8", "0"])
def test_bench_refuses_other_gpu_counts(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
