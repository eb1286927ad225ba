"""Host-side checks of bench.py's command line (no GPU is touched)."""
import os
import subprocess
import sys

from conftest import ROOT


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stdout
    assert not r.stdout.lstrip().startswith("{")   # no result line


def test_bench_refuses_a_multi_rank_launch():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True,
                       text=True, timeout=300, cwd=ROOT, env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stdout
