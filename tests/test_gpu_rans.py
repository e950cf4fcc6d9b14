"""GPU parity of the rANS lane decode (coder 1 of the interleaved-lane
container), called through the C ABI, against the CPU oracle and the
identity, bit-exact.

Containers come from both writers (the product's encoder and the oracle's);
every output buffer is framed by canary guard bands that must survive every
decode.  Expected values come only from the seeded generators, the oracle,
the golden worked example or closed forms, never from the GPU.
"""
import json
import os

import numpy as np
import pytest

from gpu_util import gpu_decode, log, to_device_aligned

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
CANARY8 = 0xA5
GUARD8 = 512


@pytest.fixture(scope="module")
def wc():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from lossless_entropy_coded_amd import wc as mod
    return mod


def _both(wc, oracle_lib, w, **kw):
    """The same input through the product's and the oracle's rANS writers."""
    return [("product", wc.encode_host([w], coder="rans", **kw)),
            ("oracle", oracle_lib.encode_lanes_rans(w, **kw))]


def gpu_decode_u8(wc, blob):
    import torch
    with wc.Plan(blob) as plan:
        assert plan.format() == (3, 1, 1)
        _, dblob = to_device_aligned(blob)
        buf = torch.full((plan.n_elems + 2 * GUARD8,), CANARY8, dtype=torch.uint8, device="cuda")
        out = buf[GUARD8:GUARD8 + plan.n_elems]
        wc.decode_u8_async(plan, dblob, out)
        torch.cuda.synchronize()
        assert bool((buf[:GUARD8] == CANARY8).all()) and bool((buf[GUARD8 + plan.n_elems:] == CANARY8).all()), \
            "decode wrote outside its output range"
        return out.cpu().numpy()


def test_rans_worked_example(wc):
    g = json.load(open(os.path.join(GOLDEN, "worked_example_rans.json")))
    w = np.array([int(v, 16) for v in g["input_bf16"]], np.uint16)
    blob = wc.encode_host([w], coder="rans")
    with wc.Plan(blob) as plan:
        assert plan.format() == (3, 0, 1)
    log(f"case: rans worked example n={w.size}")
    assert np.array_equal(gpu_decode(wc, blob), w)


@pytest.mark.parametrize("shuffle", [False, True])
def test_rans_all_bf16_patterns(wc, oracle_lib, shuffle):
    w = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if shuffle:
        w = np.random.default_rng(3).permutation(w)
    for writer, blob in _both(wc, oracle_lib, w):
        log(f"case: rans all bf16 patterns shuffle={shuffle} writer={writer}")
        assert np.array_equal(gpu_decode(wc, blob), w)


def test_rans_tiny_skewed_and_special(wc, oracle_lib):
    """Sizes around the lane block, the wave and the segment; one symbol
    (frequency 4096: the state never moves); special values; skewed and
    uniform alphabets."""
    rng = np.random.default_rng(31)
    special = np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x7F80, 0xFF80, 0x7FC1, 0xFFFF], np.uint16)
    cases = []
    for n in list(range(1, 40)) + [63, 64, 65, 511, 512, 513, 4095, 4096, 4097, 8200]:
        cases.append(rng.integers(0, 65536, n).astype(np.uint16))
        cases.append(np.full(n, 0x3F80, np.uint16))
        cases.append(special[rng.integers(0, special.size, n)])
        x = (rng.standard_normal(n).astype(np.float32) * np.float32(0.02)).view(np.uint32)
        cases.append(((x + 0x7FFF + ((x >> 16) & 1)) >> 16).astype(np.uint16))
    for i, w in enumerate(cases):
        blob = wc.encode_host([w], coder="rans") if i % 2 == 0 else oracle_lib.encode_lanes_rans(w)
        log(f"case: rans tiny #{i} n={w.size}")
        assert np.array_equal(gpu_decode(wc, blob), w), f"case {i}"


@pytest.mark.parametrize("A,M,B", [(8, 4096, 15872), (64, 1024, 4096), (8, 512, 2200), (128, 4096, 8192),
                                   (120, 3960, 15872)])
def test_rans_segment_shapes(wc, oracle_lib, A, M, B):
    from lossless_entropy_coded_amd.synth import make_workload
    wl = make_workload("block_8b", scale_rows=48)
    for writer, blob in (("product", wc.encode_host(wl.tensors(), coder="rans", group_align=A, group_max_elems=M,
                                                    seg_max_bits=B)),
                         ("oracle", oracle_lib.encode_lanes_rans(wl.bits, numels=wl.numels, group_align=A,
                                                                 group_max_elems=M, seg_max_bits=B))):
        log(f"case: rans A={A} M={M} B={B} writer={writer}")
        assert np.array_equal(gpu_decode(wc, blob), wl.bits)


@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("grid", [1, 7, 0])
def test_rans_grid_and_waves_invariance(wc, waves, grid, monkeypatch):
    from lossless_entropy_coded_amd.synth import make_workload
    monkeypatch.setenv("WC_WAVES", str(waves))
    if grid:
        monkeypatch.setenv("WC_GRID", str(grid))
    else:
        monkeypatch.delenv("WC_GRID", raising=False)
    monkeypatch.setenv("WC_DECODE_BITS", "10")     # ignored for rANS: the slot table needs 11
    wl = make_workload("attn_4k_zeros", scale_rows=64)
    blob = wc.encode_host(wl.tensors(), coder="rans")
    log(f"case: rans waves={waves} grid={grid}")
    assert np.array_equal(gpu_decode(wc, blob), wl.bits)


@pytest.mark.parametrize("name", ["block_8b", "heavy_tail_14k", "attn_4k_zeros"])
def test_rans_workload_full_size(wc, oracle_lib, name):
    """Whole workloads in one launch, against the input and the oracle (the
    full 8B-shape block: 218 M elements)."""
    from lossless_entropy_coded_amd.synth import make_workload
    wl = make_workload(name)
    blob = wc.encode_host(wl.tensors(), coder="rans")
    log(f"case: rans full {name} n={wl.n} container={blob.size}")
    got = gpu_decode(wc, blob)
    assert np.array_equal(got, wl.bits)
    log(f"case: rans full {name} oracle decode")
    assert np.array_equal(got, oracle_lib.decode(blob))


@pytest.mark.parametrize("name", ["int8_codes_8b", "int4_codes_8b"])
def test_rans_u8_code_planes(wc, oracle_lib, name):
    from lossless_entropy_coded_amd.synth import make_code_workload
    wl = make_code_workload(name, scale_rows=64)
    for writer, blob in (("product", wc.encode_u8_host(wl.tensors(), coder="rans")),
                         ("oracle", oracle_lib.encode_lanes_rans_u8(wl.codes, numels=wl.numels))):
        log(f"case: rans u8 {name} writer={writer}")
        assert np.array_equal(gpu_decode_u8(wc, blob), wl.codes)
    full = make_code_workload(name)
    blob = wc.encode_u8_host(full.tensors(), coder="rans")
    log(f"case: rans u8 full {name} n={full.n}")
    got = gpu_decode_u8(wc, blob)
    assert np.array_equal(got, full.codes)
    assert np.array_equal(got, oracle_lib.decode_u8(blob))


def test_rans_corrupted_stream_stays_in_bounds(wc):
    """Flipped stream bits and states give wrong values but no write outside
    the output and no fault (the table index is 12 bits, and a lane's word
    reads stay inside its wave's LDS region whatever the words hold)."""
    from container_view import sections
    from lossless_entropy_coded_amd.synth import make_workload
    wl = make_workload("block_8b", scale_rows=64)
    blob = wc.encode_host(wl.tensors(), coder="rans")
    s = sections(blob)
    rng = np.random.default_rng(17)
    for k in (1, 100, 5000):
        b = blob.copy()
        pos = rng.integers(0, s["stream_bits"], size=k)
        np.bitwise_xor.at(b, s["off_stream"] + pos // 8, (0x80 >> (pos % 8)).astype(np.uint8))
        log(f"case: rans corrupted flips={k}")
        assert gpu_decode(wc, b).size == wl.n
