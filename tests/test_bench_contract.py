"""The benchmark's command-line contract, checked without a GPU: it measures one GPU, and a
request for more prints one JSON line that says so and exits with status 2 (before touching
torch or the GPU)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_json_line():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    line = json.loads(res.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] or "single" in line["error"]
