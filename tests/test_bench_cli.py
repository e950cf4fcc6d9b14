"""The benchmark's command-line contract, checked without a GPU: more than
one GPU is refused with a message, and without a visible GPU the benchmark
fails loudly instead of measuring anything else."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=timeout, cwd=ROOT)


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = _run("--gpus", n)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_no_visible_gpu_fails_loudly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode != 0 and r.stdout == ""


def test_traffic_records_name_their_workload_and_source():
    sys.path.insert(0, ROOT)
    import bench
    for variant, path in bench.TRAFFIC_FILES.items():
        with open(path) as f:
            rec = json.load(f)
        assert rec["workload"] == "block_8b" and rec["traffic_bytes_per_launch"] > 0
        assert len(rec["kernel_source_sha256"]) == 64
        assert os.path.exists(os.path.join(ROOT, rec["source"])), variant
