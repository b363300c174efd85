"""bench.py's command line on the CPU: runs on more than one GPU are refused before any
GPU work, with a message and exit status 2, in every mode."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("extra", [[], ["--config", "churn"], ["--config", "prefill_30k"],
                                   ["--copy-blocks", "8"]])
def test_more_than_one_gpu_is_refused(extra):
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2", *extra], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
