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


def test_rotation_exceeds_twice_the_infinity_cache():
    """Every workload rotates at least 2 x 256 MiB of (container, output)
    copies, the small matrices included, so that a timed launch never reads a
    copy that an earlier launch left in the Infinity Cache."""
    sys.path.insert(0, ROOT)
    import bench
    from lossless_entropy_coded_amd import wc
    from lossless_entropy_coded_amd.synth import make_workload
    mall = 256 << 20
    for name in ("matrix_1k", "attn_4k_zeros"):
        wl = make_workload(name)
        per_copy = wc.encode_host(wl.tensors()).size + 2 * wl.n
        copies = bench.rotation_copies(per_copy)
        assert copies * per_copy >= 2 * mall and copies >= 2, name
    for per_copy in (1, 3_530_000, 733_000_000, 2_870_000_000):
        assert bench.rotation_copies(per_copy) * per_copy >= 2 * mall


def test_cpu_model_is_named():
    sys.path.insert(0, ROOT)
    import bench
    name = bench.cpu_model()
    assert isinstance(name, str) and name and name != "unknown"


def test_algorithmic_bytes():
    """3.36 B per element on the 8B block's shape (1 sm + L/8 stream + metadata + 2 written)."""
    sys.path.insert(0, ROOT)
    import bench
    n, bits, segs = 218_112_000, 565_226_392, 53_250
    lanes = bench.algorithmic_bytes(n, bits, segs, "lanes", 8, False)
    assert lanes == n + bits // 8 + 128 * segs + 16 * (segs + 1) + 2 * n
    chunks = bench.algorithmic_bytes(n, bits, 69_000, "chunks", 8, False)
    assert chunks == n + bits // 8 + -(-bits // 64) + 16 * 69_001 + 2 * n
    assert bench.algorithmic_bytes(n, bits, segs, "chunks", 5, False) < chunks
    assert bench.algorithmic_bytes(1000, 6000, 1, "lanes", 8, True) == 750 + 128 + 32 + 1000
