"""Pins of the oracle's packed gaps (chunks layout, header byte 10 = 5).

The DFloat11 page's auxiliary variables are a per-chunk gap here; every gap
is below the longest code (at most 23), so 5 bits hold it.  What fixes the
packed form from outside the oracle's bit loop:
- the packed section is the (separately pinned) byte gaps of the same input
  packed by numpy: gap c in bits 5c .. 5c + 4 of a little-endian bit string;
- everything else in the container equals the byte-gap container;
- the section is ceil(5 n_chunks / 8) bytes;
- identity on every workload and all 65,536 bf16 patterns, and rejection of a
  changed gap bit and of bad header bytes.
"""
import numpy as np
import pytest

from container_view import expected_metadata, sections


def _pack5(gaps: np.ndarray) -> np.ndarray:
    bits = np.unpackbits(gaps.astype(np.uint8)[:, None], axis=1, bitorder="little")[:, :5]
    return np.packbits(bits.ravel(), bitorder="little")


def _bf16(rng, n, sigma=0.02):
    x = (rng.standard_normal(n).astype(np.float32) * np.float32(sigma)).view(np.uint32)
    return ((x + 0x7FFF + ((x >> 16) & 1)) >> 16).astype(np.uint16)


CASES = [("block_8b", 16, 128, 128, 4096), ("heavy_tail_14k", 32, 128, 128, 4096), ("attn_4k_zeros", 64, 3, 4, 8),
         ("matrix_1k", None, 2, 64, 64), ("block_70b", 4, 128, 8, 64)]


@pytest.mark.parametrize("name,rows,G,A,M", CASES)
def test_packed_gaps_are_the_byte_gaps_packed(oracle_lib, name, rows, G, A, M):
    from lossless_entropy_coded_amd.synth import make_workload
    wl = make_workload(name, scale_rows=rows) if rows else make_workload(name)
    kw = dict(numels=wl.numels, chunks_per_group=G, group_align=A, group_max_elems=M)
    b8 = oracle_lib.encode(wl.bits, **kw)
    b5 = oracle_lib.encode(wl.bits, gap_bits=5, **kw)
    s8, s5 = sections(b8), sections(b5)
    assert s8["gap_bits"] == 8 and s5["gap_bits"] == 5 and b5[10] == 5 and b8[10] == 0
    nc = s8["n_chunks"]
    # the byte gaps are the numpy restatement's (pinned in test_oracle_pins)
    exps = ((wl.bits >> 7) & 0xFF).astype(np.int64)
    _, gap, groups = expected_metadata(exps, s8["code_len"], G, A, M)
    assert np.array_equal(s8["gap"], gap) and np.array_equal(s8["groups"], groups)
    assert np.array_equal(s5["gap_packed"], _pack5(s8["gap"])[:(5 * nc + 7) // 8])
    assert s5["off_stream"] - s5["off_gap"] >= (5 * nc + 7) // 8
    for k in ("code_len", "tensors", "groups", "stream", "sm"):
        assert np.array_equal(s8[k], s5[k]), k
    assert s8["stream_bits"] == s5["stream_bits"] and s8["n_groups"] == s5["n_groups"]
    assert b5.size <= b8.size
    assert np.array_equal(oracle_lib.decode(b5), wl.bits)


@pytest.mark.parametrize("shuffle", [False, True])
def test_packed_gaps_all_bf16_patterns(oracle_lib, shuffle):
    w = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if shuffle:
        w = np.random.default_rng(4).permutation(w)
    b5 = oracle_lib.encode(w, gap_bits=5)
    s5 = sections(b5)
    assert (s5["gap"] == 0).all()                  # every code is 8 bits: chunks start on codewords
    out, rep = oracle_lib.decode(b5, with_report=True)
    assert np.array_equal(out, w) and rep["gap_bits"] == 5


@pytest.mark.parametrize("n", [0, 1, 7, 100, 5000, 70_001])
def test_packed_gaps_round_trip_sizes(oracle_lib, n):
    w = _bf16(np.random.default_rng(n), n)
    for G, A, M in ((128, 128, 4096), (3, 8, 64), (1, 1, 8)):
        b5 = oracle_lib.encode(w, gap_bits=5, chunks_per_group=G, group_align=A, group_max_elems=M)
        assert np.array_equal(oracle_lib.decode(b5), w)
        s8 = sections(oracle_lib.encode(w, chunks_per_group=G, group_align=A, group_max_elems=M))
        assert np.array_equal(sections(b5)["gap"], s8["gap"])


def test_packed_gaps_reject_corruption(oracle_lib):
    w = _bf16(np.random.default_rng(9), 30_000)
    b5 = oracle_lib.encode(w, gap_bits=5, chunks_per_group=16, group_align=64, group_max_elems=1024)
    s5 = sections(b5)
    assert oracle_lib.decode_status(b5) == 0
    nz = np.nonzero(s5["gap"])[0]
    c = int(nz[len(nz) // 2])                      # a chunk with a non-zero gap
    for j in range(5):
        b = b5.copy()
        bit = 5 * c + j
        b[s5["off_gap"] + bit // 8] ^= np.uint8(1 << (bit % 8))
        assert oracle_lib.decode_status(b) == -9, j    # ORC_E_GAP
    for off, val in ((10, 6), (10, 8), (11, 1)):
        b = b5.copy()
        b[off] = val
        assert oracle_lib.decode_status(b) == -2, (off, val)
    with pytest.raises(oracle_lib.OracleError):
        oracle_lib.encode(w, gap_bits=6)
