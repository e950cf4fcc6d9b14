"""Pins of the oracle's rANS coder in the interleaved-lane layout (coder 1).

The Llama2-7B page names ANS (Asymmetric Numeral Systems) as its hardware
coder, and the LazyWeights page compares a Huffman and an rANS decoder.  What
fixes the oracle's rANS from outside it:
- a hand-derived worked example (tests/golden/worked_example_rans.json) that
  fixes the state range, the symbol order of the cumulative frequencies, the
  renormalisation and the word order;
- the rate of every lane against the bounds that ANS's arithmetic proves:
  with x in [2^16, 2^32), a lane of symbols s_i takes at most
  32 + sum(12 - log2 f + 0.0875) bits and at least 16 + sum(12 - log2 f - 0.0931);
- the quantized frequencies: they sum to 2^12, are non-zero exactly for the
  present symbols, and their cross-entropy is within 0.01 bit of the entropy
  on the workloads;
- the identity on every workload and on all 65,536 bf16 patterns, and the
  rejection of corrupted states, words, frequencies and offsets.
"""
import json
import math
import os

import numpy as np
import pytest

from container_view import sections

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(rng, n, sigma=0.02):
    x = (rng.standard_normal(n).astype(np.float32) * np.float32(sigma)).view(np.uint32)
    return ((x + 0x7FFF + ((x >> 16) & 1)) >> 16).astype(np.uint16)


def test_rans_worked_example(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "worked_example_rans.json")))
    w = np.array([int(v, 16) for v in g["input_bf16"]], np.uint16)
    blob = oracle_lib.encode_lanes_rans(w)
    s = sections(blob)
    assert s["version"] == 3 and s["coder"] == g["coder"]
    assert {str(k): int(s["freq"][k]) for k in range(256) if s["freq"][k]} == g["frequencies"]
    assert s["stream_bits"] == g["stream_bits"]
    assert [f"{b:02X}" for b in s["stream"][:4]] == g["stream_bytes_hex"]
    assert s["groups"].tolist() == g["segments"]
    assert s["lane_off"][0, 0] == g["lane_off_first"] and (s["lane_off"][0, 1:] == g["lane_off_rest"]).all()
    out, rep = oracle_lib.decode(blob, with_report=True)
    assert np.array_equal(out, w) and rep["coder"] == 1


def _lane_symbols(e, segs):
    """(segment, lane) -> symbols of that lane, in lane order."""
    for g in range(len(segs) - 1):
        a, b = int(segs[g, 0]), int(segs[g + 1, 0])
        idx = np.arange(b - a)
        lane = (idx // 8) % 64
        for j in range(64):
            yield g, j, e[a:b][lane == j]


@pytest.mark.parametrize("name,rows", [("heavy_tail_14k", 16), ("block_8b", 8), ("attn_4k_zeros", 32)])
def test_rans_rate_bounds_and_frequencies(oracle_lib, name, rows):
    from lossless_entropy_coded_amd.synth import make_workload
    wl = make_workload(name, scale_rows=rows)
    blob = oracle_lib.encode_lanes_rans(wl.bits, numels=wl.numels)
    s = sections(blob)
    f = s["freq"].astype(np.int64)
    e = ((wl.bits >> 7) & 0xFF).astype(np.int64)
    hist = np.bincount(e, minlength=256)
    assert f.sum() == 4096 and ((f > 0) == (hist > 0)).all()
    p = hist[hist > 0] / e.size
    H = -(p * np.log2(p)).sum()
    cross = -(p * np.log2(f[hist > 0] / 4096)).sum()
    assert H <= cross < H + 0.01
    segs = s["groups"].astype(np.int64)
    cost = 12 - np.log2(np.maximum(f, 1).astype(np.float64))
    k = 0
    for g, j, sym in _lane_symbols(e, segs):
        start = int(s["lane_off"][g, j])
        end = int(s["lane_off"][g, j + 1]) if j < 63 else int(segs[g + 1, 1] - segs[g, 1])
        bits = end - start
        if sym.size == 0:
            assert bits == 0
            continue
        c = cost[sym].sum()
        assert bits % 16 == 0
        assert 16 + c - 0.0931 * sym.size - 1e-6 <= bits <= 32 + c + 0.0875 * sym.size + 1e-6
        k += 1
    assert k > 0
    assert np.array_equal(oracle_lib.decode(blob), wl.bits)


@pytest.mark.parametrize("shuffle", [False, True])
def test_rans_all_bf16_patterns(oracle_lib, shuffle):
    w = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if shuffle:
        w = np.random.default_rng(3).permutation(w)
    blob = oracle_lib.encode_lanes_rans(w)
    s = sections(blob)
    assert (s["freq"] == 16).all()                  # every exponent 256 times: uniform
    out, rep = oracle_lib.decode(blob, with_report=True)
    assert np.array_equal(out, w)
    # uniform frequencies: exactly 8 bits of information per symbol
    assert 8 * 65536 <= s["stream_bits"] <= 8 * 65536 + 32 * 64 * s["n_groups"]


@pytest.mark.parametrize("n,A,M,B", [(0, 128, 4096, 15872), (1, 128, 4096, 15872), (7, 8, 64, 2200),
                                     (5000, 8, 512, 2200), (100_003, 64, 1024, 6000), (70_000, 128, 4096, 15872)])
def test_rans_round_trip_shapes(oracle_lib, n, A, M, B):
    w = _bf16(np.random.default_rng(n + 7), n)
    blob = oracle_lib.encode_lanes_rans(w, group_align=A, group_max_elems=M, seg_max_bits=B)
    assert np.array_equal(oracle_lib.decode(blob), w)
    s = sections(blob)
    assert (s["groups"][1:, 1] - s["groups"][:-1, 1] <= B).all()


def test_rans_u8_round_trip(oracle_lib):
    from lossless_entropy_coded_amd.synth import make_code_workload
    wl = make_code_workload("int8_codes_8b", scale_rows=16)
    blob = oracle_lib.encode_lanes_rans_u8(wl.codes, numels=wl.numels)
    out, rep = oracle_lib.decode_u8(blob, with_report=True)
    assert np.array_equal(out, wl.codes) and rep["coder"] == 1 and rep["elem_kind"] == 1


def test_rans_special_values(oracle_lib):
    special = np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x7F80, 0xFF80, 0x7FC1, 0xFFFF], np.uint16)
    rng = np.random.default_rng(1)
    for n in (1, 2, 9, 513, 4100):
        w = special[rng.integers(0, special.size, n)]
        assert np.array_equal(oracle_lib.decode(oracle_lib.encode_lanes_rans(w)), w)
    one = np.full(3000, 0x3F80, np.uint16)          # a single symbol: frequency 4096, no bits per symbol
    s = sections(oracle_lib.encode_lanes_rans(one))
    assert s["freq"][127] == 4096
    assert np.array_equal(oracle_lib.decode(oracle_lib.encode_lanes_rans(one)), one)


def test_rans_rejects_corruption(oracle_lib):
    w = _bf16(np.random.default_rng(5), 20_000)
    blob = oracle_lib.encode_lanes_rans(w, group_align=64, group_max_elems=1024, seg_max_bits=6000)
    assert oracle_lib.decode_status(blob) == 0
    s = sections(blob)
    h = {k: int(v) for k, v in s.items() if isinstance(v, (int, np.integer))}

    def status_after(mutate):
        b = blob.copy()
        mutate(b)
        return oracle_lib.decode_status(b)

    st = h["off_stream"]
    assert status_after(lambda b: b.__setitem__(st + 1, b[st + 1] ^ 0x01)) == -7       # lane 0's state
    assert status_after(lambda b: b.__setitem__(st + 200, b[st + 200] ^ 0x40)) != 0     # some word
    fo = h["off_len"]
    sym = int(np.argmax(s["freq"]))
    assert status_after(lambda b: b.__setitem__(fo + 2 * sym, b[fo + 2 * sym] ^ 1)) == -5  # sum != 4096
    lo = h["off_gap"]
    assert status_after(lambda b: b.__setitem__(slice(lo + 2, lo + 4), [16, 0])) == -10   # lane 1 offset
    assert status_after(lambda b: b.__setitem__(125, 2)) == -2                            # unknown coder
    assert status_after(lambda b: b.__setitem__(8, 11)) == -2                             # P must be 12


def test_rans_cost_restatement_closed_forms():
    """The per-symbol cost bound in eighths at the ends and at a power of two."""
    from container_view import rans_cost_eighths
    assert rans_cost_eighths(4096) == 1          # log2 f = 12: no bits, plus the eighth of margin
    assert rans_cost_eighths(1) == 97            # 12 bits
    assert rans_cost_eighths(2048) == 9          # 1 bit
    assert rans_cost_eighths(3) == 97 - 12       # 8 log2 3 = 12.68...
    for f in range(1, 4097):
        c = rans_cost_eighths(f)
        assert c - 1 >= 8 * (12 - math.log2(f)) - 1e-9 and c - 2 < 8 * (12 - math.log2(f)) + 1e-9


@pytest.mark.parametrize("name,rows,A,M,B", [
    ("block_8b", 8, 128, 4096, 15872),            # the default: M binds
    ("heavy_tail_14k", 16, 128, 4096, 15872),
    ("attn_4k_zeros", 32, 64, 4096, 6000),        # the bound binds
    ("block_8b", 4, 8, 512, 2200),                # tiny B: one or a few blocks per segment
    ("heavy_tail_14k", 8, 120, 3840, 9000),
])
def test_rans_frequencies_and_segments_restated(oracle_lib, name, rows, A, M, B):
    """The oracle's quantized frequencies and segment cut equal numpy
    restatements of the rules (tie breaks included): a cut one block early or
    late, or a unit of excess taken from the wrong symbol, fails here."""
    from container_view import expected_rans_freqs, expected_rans_segment_elems
    from lossless_entropy_coded_amd.synth import make_workload
    wl = make_workload(name, scale_rows=rows)
    blob = oracle_lib.encode_lanes_rans(wl.bits, numels=wl.numels, group_align=A, group_max_elems=M,
                                        seg_max_bits=B)
    s = sections(blob)
    e = ((wl.bits >> 7) & 0xFF).astype(np.int64)
    freq = expected_rans_freqs(np.bincount(e, minlength=256))
    assert np.array_equal(s["freq"].astype(np.int64), freq)
    elems = expected_rans_segment_elems(e, freq, A, M, B)
    assert np.array_equal(s["groups"][:, 0], elems)
    assert s["n_groups"] == elems.size - 1 > 1


def test_rans_frequency_tie_rules():
    """Hand-worked cases of the quantization's two tie rules."""
    from container_view import expected_rans_freqs
    # 3 symbols of equal count 1 among n = 3: floor(4096/3) = 1365 each, sum 4095;
    # the shortfall of 1 goes to the lowest of the equally frequent symbols
    h = np.zeros(256, np.int64)
    h[[5, 9, 200]] = 1
    f = expected_rans_freqs(h)
    assert f[5] == 1366 and f[9] == 1365 and f[200] == 1365
    # two frequent symbols and 253 rare ones, n = 20,000,253: floor(4096 * 10^7 / n) = 2047
    # each, every rare symbol is lifted to 1, so the sum is 4347 and 251 units are taken,
    # one at a time from the largest frequency (the lower symbol first on a tie):
    # 126 from symbol 0 and 125 from symbol 1
    h = np.zeros(256, np.int64)
    h[0] = h[1] = 10_000_000
    h[2:255] = 1
    f = expected_rans_freqs(h)
    assert f.sum() == 4096 and (f[2:255] == 1).all() and f[255] == 0
    assert f[0] == 2047 - 126 and f[1] == 2047 - 125


def test_rans_oracle_frequency_ties(oracle_lib):
    """The oracle on a histogram whose quantization needs both tie rules:
    exponents 0 and 1 seen 100,000 times each and 253 others once, n = 200,253:
    floor(4096 * 10^5 / n) = 2045 each, the rare ones lifted to 1, sum 4343,
    so 247 units are taken alternately, 124 from exponent 0 (lower first) and
    123 from exponent 1."""
    e = np.concatenate([np.zeros(100_000, np.uint16), np.ones(100_000, np.uint16), np.arange(2, 255, dtype=np.uint16)])
    w = (np.random.default_rng(4).permutation(e) << 7).astype(np.uint16)
    s = sections(oracle_lib.encode_lanes_rans(w))
    f = s["freq"].astype(np.int64)
    assert f[0] == 2045 - 124 and f[1] == 2045 - 123 and (f[2:255] == 1).all() and f[255] == 0
