"""GPU parity of the chunks-layout decode with packed 5-bit gaps (header byte
10 = 5), called through the C ABI, against the CPU oracle and the identity,
bit-exact, from both writers.  Every output buffer is framed by canary guard
bands that must survive every decode."""
import numpy as np
import pytest

from gpu_util import gpu_decode, log
from test_gpu_parity import _fib_alphabet, _many_rare_exponents

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wc():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from lossless_entropy_coded_amd import wc as mod
    return mod


def _both(wc, oracle_lib, w, numels=None, **kw):
    tensors = [w] if numels is None else np.split(w, np.cumsum(numels)[:-1])
    return [("product", wc.encode_host(tensors, layout="chunks", gap_bits=5, **kw)),
            ("oracle", oracle_lib.encode(w, numels=numels, gap_bits=5,
                                         chunks_per_group=kw.get("chunks_per_group", wc.GROUP_CHUNKS),
                                         group_align=kw.get("group_align", wc.GROUP_ALIGN),
                                         group_max_elems=kw.get("group_max_elems", wc.GROUP_MAX_ELEMS)))]


@pytest.mark.parametrize("shuffle", [False, True])
def test_gap5_all_bf16_patterns(wc, oracle_lib, shuffle):
    w = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if shuffle:
        w = np.random.default_rng(3).permutation(w)
    for writer, blob in _both(wc, oracle_lib, w):
        log(f"case: gap5 all patterns shuffle={shuffle} writer={writer}")
        assert np.array_equal(gpu_decode(wc, blob), w)


def test_gap5_tiny_special_and_long_codes(wc, oracle_lib):
    rng = np.random.default_rng(55)
    special = np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x7F80, 0xFF80, 0x7FC1, 0xFFFF], np.uint16)
    cases = [np.zeros(0, np.uint16)]
    for n in list(range(1, 24)) + [63, 64, 65, 255, 256, 257, 4095, 4096, 4097]:
        cases.append(special[rng.integers(0, special.size, size=n)])
        cases.append(rng.integers(0, 65536, size=n, dtype=np.uint16))
    cases += [_fib_alphabet([100] * 63 + [124]), _fib_alphabet([124] * 10), _many_rare_exponents()]
    for i, w in enumerate(cases):
        writer, blob = _both(wc, oracle_lib, w)[i % 2]
        log(f"case: gap5 #{i} n={w.size} writer={writer}")
        assert np.array_equal(gpu_decode(wc, blob), w), f"case {i}"


@pytest.mark.parametrize("align", [8, 64, 120, 128, 256])
def test_gap5_group_block_sizes(wc, oracle_lib, align):
    """Groups start at every chunk offset, so lanes read their two gaps from
    every bit position of the packed section."""
    from lossless_entropy_coded_amd.synth import make_workload
    wl = make_workload("heavy_tail_14k", scale_rows=256)
    M = wc.GROUP_MAX_ELEMS // align * align
    for writer, blob in _both(wc, oracle_lib, wl.bits, numels=wl.numels, group_align=align, group_max_elems=M):
        log(f"case: gap5 group_align={align} writer={writer}")
        assert np.array_equal(gpu_decode(wc, blob), wl.bits)


@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("grid", [1, 7, 0])
def test_gap5_grid_and_waves(wc, waves, grid, monkeypatch):
    from lossless_entropy_coded_amd.synth import make_workload
    monkeypatch.setenv("WC_WAVES", str(waves))
    if grid:
        monkeypatch.setenv("WC_GRID", str(grid))
    else:
        monkeypatch.delenv("WC_GRID", raising=False)
    wl = make_workload("attn_4k_zeros", scale_rows=64)
    blob = wc.encode_host(wl.tensors(), layout="chunks", gap_bits=5)
    log(f"case: gap5 waves={waves} grid={grid}")
    assert np.array_equal(gpu_decode(wc, blob), wl.bits)


@pytest.mark.parametrize("name", ["block_8b", "heavy_tail_14k"])
def test_gap5_workload_full_size(wc, oracle_lib, name):
    from lossless_entropy_coded_amd.synth import make_workload
    wl = make_workload(name)
    blob = wc.encode_host(wl.tensors(), layout="chunks", gap_bits=5)
    log(f"case: gap5 full {name} n={wl.n} container={blob.size}")
    got = gpu_decode(wc, blob)
    assert np.array_equal(got, wl.bits)
    log(f"case: gap5 full {name} oracle decode")
    assert np.array_equal(got, oracle_lib.decode(blob))


def test_gap5_corrupted_stream_and_gaps_stay_in_bounds(wc):
    """Flipped stream bits, and packed gaps changed to other values below the
    longest code (which wc_plan accepts): wrong output, no write outside it."""
    from container_view import sections
    from lossless_entropy_coded_amd.synth import make_workload
    wl = make_workload("matrix_1k", scale_rows=256)
    blob = wc.encode_host(wl.tensors(), layout="chunks", gap_bits=5)
    s = sections(blob)
    rng = np.random.default_rng(13)
    for k in (1, 1000):
        b = blob.copy()
        pos = rng.integers(0, s["stream_bits"], size=k)
        np.bitwise_xor.at(b, s["off_stream"] + pos // 8, (0x80 >> (pos % 8)).astype(np.uint8))
        log(f"case: gap5 corrupted stream flips={k}")
        assert gpu_decode(wc, b).size == wl.n
    b = blob.copy()
    longest = int(s["code_len"].max())
    for c in range(0, int(s["n_chunks"]) - 1, 7):
        g = int(rng.integers(0, longest))
        for j in range(5):
            bit = 5 * c + j
            byte = s["off_gap"] + bit // 8
            b[byte] = (b[byte] & ~np.uint8(1 << (bit % 8))) | np.uint8(((g >> j) & 1) << (bit % 8))
    log("case: gap5 rewritten gaps")
    assert gpu_decode(wc, b).size == wl.n
