"""GPU parity of the interleaved-lane decode kernel (container version 3),
called through the C ABI, against the CPU oracle and the identity,
bit-exact.

Every output buffer is framed by canary guard bands that must survive every
decode.  Expected values come only from the seeded generators, the oracle or
closed forms, never from the GPU.
"""
import os

import numpy as np
import pytest

from gpu_util import GuardedOutput, gpu_decode, log, to_device_aligned
from test_gpu_parity import _fib_alphabet, _many_rare_exponents

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wc():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from lossless_entropy_coded_amd import wc as mod
    return mod


@pytest.fixture
def env_knob():
    saved = {}

    def setter(name, value):
        if name not in saved:
            saved[name] = os.environ.get(name)
        if value is None:
            os.environ.pop(name, None)
        else:
            os.environ[name] = str(value)
    yield setter
    for k, v in saved.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v


def _lanes(wc, tensors, **kw):
    return wc.encode_host(tensors, layout="lanes", **kw)


def test_lanes_worked_example(wc):
    w = np.array([0x3C80, 0x3C00, 0x3C80, 0x3B80, 0x3C80, 0x3D00, 0x3C00, 0x3C80], np.uint16)
    log("case: lanes worked example n=8")
    assert np.array_equal(gpu_decode(wc, _lanes(wc, [w])), w)


@pytest.mark.parametrize("shuffle", [False, True])
def test_lanes_all_bf16_patterns(wc, oracle_lib, shuffle):
    w = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if shuffle:
        w = np.random.default_rng(99).permutation(w)
    for writer in ("product", "oracle"):
        blob = _lanes(wc, [w]) if writer == "product" else oracle_lib.encode_lanes(w)
        log(f"case: lanes all 65536 patterns shuffle={shuffle} writer={writer}")
        assert np.array_equal(gpu_decode(wc, blob), w)


def test_lanes_tiny_and_special_sequences(wc, oracle_lib):
    """Every element count around the lane-block, lane and segment sizes,
    special values, random patterns and constant input."""
    rng = np.random.default_rng(2025)
    special = np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x7F80, 0xFF80, 0x7FC1, 0xFFFF, 0x3F80, 0xBF80],
                       np.uint16)
    cases = [np.zeros(0, np.uint16), np.array([0x1234], np.uint16)]
    for n in list(range(1, 40)) + [63, 64, 65, 127, 128, 129, 511, 512, 513, 520, 4095, 4096, 4097, 8200]:
        cases.append(special[rng.integers(0, special.size, size=n)])
        cases.append(rng.integers(0, 65536, size=n, dtype=np.uint16))
        cases.append(np.full(n, 0x3C00, np.uint16))
    for i, w in enumerate(cases):
        log(f"case: lanes tiny #{i} n={w.size}")
        blob = _lanes(wc, [w]) if i % 2 == 0 else oracle_lib.encode_lanes(w)
        assert np.array_equal(gpu_decode(wc, blob), w), f"case {i} n={w.size}"


@pytest.mark.parametrize("prefix", [[100] * 63 + [124], [124] * 10, [123, 124] * 8, []])
def test_lanes_long_codes(wc, oracle_lib, prefix):
    """Code lengths up to 24 bits (the long-code path), both writers; with a
    small bit cap, segments are cut by bits rather than elements."""
    w = _fib_alphabet(prefix)
    for writer in ("product", "oracle"):
        for B in (15872, 128 * 24):
            blob = (_lanes(wc, [w], seg_max_bits=B) if writer == "product"
                    else oracle_lib.encode_lanes(w, seg_max_bits=B))
            log(f"case: lanes fib alphabet prefix_len={len(prefix)} writer={writer} B={B} n={w.size}")
            assert np.array_equal(gpu_decode(wc, blob), w)


@pytest.mark.parametrize("bits", [(12, 11), (12, 10)])
def test_lanes_many_long_code_prefixes(wc, env_knob, bits):
    w = _many_rare_exponents()
    blob = _lanes(wc, [w])
    env_knob("WC_COUNT_BITS", bits[0])
    env_knob("WC_DECODE_BITS", bits[1])
    log(f"case: lanes many rare exponents n={w.size} table bits={bits}")
    with wc.Plan(blob) as plan:
        assert plan.stats()["decode_bits"] == bits[1]
        assert np.array_equal(gpu_decode(wc, blob, plan=plan), w)


@pytest.mark.parametrize("decode_bits", [11, 10])
@pytest.mark.parametrize("grid", [1, 7, 16, 0])
@pytest.mark.parametrize("waves", [4, 8])
def test_lanes_table_width_and_grid_invariance(wc, env_knob, decode_bits, grid, waves):
    from lossless_entropy_coded_amd.synth import make_workload
    wl = make_workload("heavy_tail_14k", scale_rows=512)
    blob = _lanes(wc, wl.tensors())
    env_knob("WC_COUNT_BITS", 12)
    env_knob("WC_DECODE_BITS", decode_bits)
    env_knob("WC_GRID", grid or None)
    env_knob("WC_WAVES", waves)
    log(f"case: lanes heavy_tail rows=512 decode bits={decode_bits} grid={grid} waves={waves}")
    with wc.Plan(blob) as plan:
        st = plan.stats()
        assert st["decode_bits"] == decode_bits
        if grid:
            assert st["grid"] == grid
        assert np.array_equal(gpu_decode(wc, blob, plan=plan), wl.bits)


@pytest.mark.parametrize("A,M,B", [(8, 4096, 15872), (64, 1024, 4096), (120, 3960, 15872), (8, 512, 500),
                                   (256, 4096, 8192)])
@pytest.mark.parametrize("writer", ["product", "oracle"])
def test_lanes_segment_shapes(wc, oracle_lib, A, M, B, writer):
    """Block sizes, element caps and bit caps: segments start on any
    8-element boundary, hold from one block to 4096 elements, and their first
    bit sits anywhere in a 16-byte window."""
    from lossless_entropy_coded_amd.synth import make_workload
    wl = make_workload("heavy_tail_14k", scale_rows=256)
    if writer == "product":
        blob = _lanes(wc, wl.tensors(), group_align=A, group_max_elems=M, seg_max_bits=B)
    else:
        blob = oracle_lib.encode_lanes(wl.bits, numels=wl.numels, group_align=A, group_max_elems=M,
                                       seg_max_bits=B)
    log(f"case: lanes A={A} M={M} B={B} writer={writer}")
    assert np.array_equal(gpu_decode(wc, blob), wl.bits)


@pytest.mark.parametrize("name", ["matrix_1k", "attn_4k_zeros", "block_8b", "heavy_tail_14k", "block_70b"])
def test_lanes_workload_full_size(wc, oracle_lib, name):
    """Full-size workloads, one launch each, in the benchmark's launch configuration."""
    import torch
    from lossless_entropy_coded_amd.synth import make_workload
    wl = make_workload(name)
    blob = _lanes(wc, wl.tensors())
    log(f"case: lanes full {name} n={wl.n} container={blob.size}")
    with wc.Plan(blob) as plan:
        _, dblob = to_device_aligned(blob)
        out = GuardedOutput(wl.n)
        wc.decode_async(plan, dblob, out.out)
        torch.cuda.synchronize()
        assert out.guards_intact()
        ref = torch.from_numpy(wl.bits.view(np.int16)).cuda()
        assert torch.equal(out.out, ref), "GPU decode differs from the input weights"
        del ref
        if wl.n <= 300_000_000:
            log(f"case: lanes full {name} oracle decode")
            assert np.array_equal(out.host(), oracle_lib.decode(blob))


def test_lanes_corrupted_stream_stays_in_bounds(wc):
    """Valid metadata, garbage bits or lane offsets that are not where the
    lanes' bits begin: the output may be wrong, but nothing is written outside
    [out, out + n)."""
    from container_view import sections
    from lossless_entropy_coded_amd.synth import make_workload
    wl = make_workload("matrix_1k", scale_rows=256)
    blob = _lanes(wc, wl.tensors())
    s = sections(blob)
    rng = np.random.default_rng(4)
    nbytes = (s["stream_bits"] + 7) // 8
    variants = []
    for k in (1, 10, 1000):
        b = blob.copy()
        pos = rng.integers(0, s["stream_bits"], size=k)
        np.bitwise_xor.at(b, s["off_stream"] + pos // 8, (0x80 >> (pos % 8)).astype(np.uint8))
        variants.append(("flip%d" % k, b))
    for fill in (0xFF, 0x00):
        b = blob.copy()
        b[s["off_stream"]:s["off_stream"] + nbytes - 1] = fill
        variants.append(("fill%02x" % fill, b))
    # lane offsets moved (still non-decreasing and inside the segment)
    for shift in (1, 7):
        b = blob.copy()
        lo = s["lane_off"].astype(np.int64).copy()
        seg_bits = (s["groups"][1:, 1] - s["groups"][:-1, 1]).astype(np.int64)
        lo[:, 1:] = np.minimum(lo[:, 1:] + shift, seg_bits[:, None])
        lo = np.maximum.accumulate(lo, axis=1)
        b[s["off_gap"]:s["off_gap"] + lo.size * 2] = lo.astype(np.uint16).ravel().view(np.uint8)
        variants.append(("lane-offsets+%d" % shift, b))
    for tag, b in variants:
        log(f"case: lanes corrupted {tag}")
        got = gpu_decode(wc, b)          # asserts the guard bands
        assert got.size == wl.n


def test_lanes_plan_reuse_across_streams(wc):
    import torch
    from lossless_entropy_coded_amd.synth import make_workload
    wl = make_workload("attn_4k_zeros", scale_rows=1024)
    blob = _lanes(wc, wl.tensors())
    ref = torch.from_numpy(wl.bits.view(np.int16)).cuda()
    log("case: lanes two streams, repeated decodes")
    with wc.Plan(blob) as plan:
        _, dblob = to_device_aligned(blob)
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        outs = [GuardedOutput(wl.n) for _ in range(4)]
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            wc.decode_async(plan, dblob, o.out, stream=(s1 if i % 2 else s2))
        torch.cuda.synchronize()
        for o in outs:
            assert o.guards_intact() and torch.equal(o.out, ref)
