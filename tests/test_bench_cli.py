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


def _sample_line():
    import json
    path = os.path.join(ROOT, "profiles", "bench_block_8b_default.md")
    text = open(path).read()
    return json.loads(text.split("```json\n", 1)[1].split("\n```", 1)[0])


def test_committed_bench_line_has_the_contract_fields():
    """The committed sample of the default run's line carries every field of
    the contract and of this benchmark's records."""
    d = _sample_line()
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "layouts", "e2e"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["higher_is_better"] is True and d["scaling"] == "weak" and d["unit"] == "GB/s"
    assert d["vs_baseline"] is None and d["data"].startswith("synthetic")
    assert d["config"]["workload"].startswith("block_8b") and d["config"]["bit_exact"] is True
    assert d["config"]["timed_outputs_checked"] >= 2 and d["config"]["rotated_bytes"] >= 1 << 30
    r = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "algorithmic_bytes_per_launch", "kernel_avg_ms",
              "launch_us", "stream_ref", "frac_of_stream_ref"):
        assert k in r, k
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] >= 1 and c["cpu_model"] and c["sample"] and c["value"] > 0
    for k in ("ms", "frac", "bit_exact", "frac_of_stream_ref", "traffic"):
        assert k in d["layouts"]["chunks"], k
    for k in ("arm_a_decode_plus_gemv_ms", "arm_b_uncompressed_gemv_ms", "arm_c_fused_decode_gemv_ms",
              "decode_only_ms", "ratio_c_over_b", "decode_frac_of_stream_ref"):
        assert k in d["e2e"], k
    assert d["e2e"]["outputs_bit_identical_a_b"] and d["e2e"]["decoded_weights_bit_exact"]
    assert d["e2e"]["fused_within_bound"]


def test_committed_bench_line_arithmetic():
    """value, roofline and ratios in the committed sample follow from its own
    timings and byte counts."""
    d = _sample_line()
    r, cfg = d["roofline"], d["config"]
    n = cfg["n_elems"]
    assert abs(d["value"] - 2 * n / (d["ms_per_step"] * 1e-3) / 1e9) <= 0.01 * d["value"]
    achieved = r["algorithmic_bytes_per_launch"] / (r["kernel_avg_ms"] * 1e-3) / 1e9
    assert abs(r["achieved"] - achieved) <= 0.5
    assert abs(r["frac"] - r["achieved"] / r["peak"]) <= 1e-4
    assert abs(r["frac_of_stream_ref"] - r["achieved"] / r["stream_ref"]["GBps"]) <= 1e-3
    sref = r["stream_ref"]
    assert abs(sref["GBps"] - (sref["read_bytes"] + sref["write_bytes"]) / (sref["ms"] * 1e-3) / 1e9) <= 0.01 * sref["GBps"]
    # measured HBM traffic within 5% above the algorithmic bytes
    assert 1.0 <= r["traffic"] / r["algorithmic_bytes_per_launch"] <= 1.05
    # the algorithmic reads are the container's sections the decode needs:
    # all of it but the header, code lengths, tensor table and padding
    reads = r["algorithmic_bytes_per_launch"] - 2 * n
    assert 0.99 * cfg["container_bytes"] <= reads <= cfg["container_bytes"]
    e = d["e2e"]
    assert abs(e["ratio_c_over_b"] - e["arm_c_fused_decode_gemv_ms"] / e["arm_b_uncompressed_gemv_ms"]) <= 2e-3
    assert abs(e["ratio_a_over_b"] - e["arm_a_decode_plus_gemv_ms"] / e["arm_b_uncompressed_gemv_ms"]) <= 2e-3


def test_packed_gaps_have_no_traffic_record():
    """The chunks layout's record is for byte gaps; packed gaps change the
    bytes moved, so no recorded traffic applies to them."""
    sys.path.insert(0, ROOT)
    import bench
    assert bench.variant_of("chunks", "huffman", 5) == "chunks_gap5"
    assert bench.recorded_traffic("block_8b", "chunks", "huffman", 5) is None
    assert bench.variant_of("lanes", "rans", 8) == "lanes_rans"
