"""bench.py's contract checks that need no GPU: one GPU only, and the argument defaults."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1", "--warmup", "0"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout.strip() == ""


def test_defaults_time_the_largest_single_gpu_workload():
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert 'ap.add_argument("--config", type=int, default=2,' in src  # the 32k latent prefill
    assert 'ap.add_argument("--gpus", type=int, default=1)' in src
