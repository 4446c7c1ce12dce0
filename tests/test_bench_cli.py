"""bench.py's contract checks that need no GPU: more than one GPU is refused with a message."""
import os
import subprocess
import sys


def test_bench_refuses_more_than_one_gpu(repo_root):
    r = subprocess.run([sys.executable, os.path.join(repo_root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one-GPU" in r.stderr and "no multi-GPU path" in r.stderr
    assert r.stdout == ""
