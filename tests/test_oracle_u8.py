"""Pins of the oracle's symbol-plane coder for 8-bit codes (element kind u8).

Planes of quantized integer codes (the LazyWeights page's setting) are coded
byte by byte with the same canonical code and lane layout as the bf16
exponents, with no raw plane.  What fixes it from outside the oracle:
- a hand-derived worked example (tests/golden/worked_example_u8.json);
- all 256 byte values 256 times each: every code is 8 bits, the code is the
  byte itself, and the stream is the bytes permuted into lane order;
- equality with the (separately pinned) bf16 kind: bf16 words whose exponent
  field is the code and whose other bits are zero give the same code lengths,
  segment table, lane offsets and stream bytes;
- the generator of the stand-in codes against the closed form of a rounded,
  clipped Gaussian (chi-squared), and the entropy bound on its planes;
- rejection of a wrong element kind.
"""
import json
import math
import os

import numpy as np
import pytest

from container_view import lane_permutation, sections

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_u8_worked_example(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "worked_example_u8.json")))
    c = np.array(g["codes"], np.uint8)
    blob = oracle_lib.encode_lanes_u8(c)
    s = sections(blob)
    assert s["version"] == 3 and s["elem_kind"] == g["elem_kind"]
    assert {str(k): int(s["code_len"][k]) for k in range(256) if s["code_len"][k]} == g["code_lengths"]
    assert s["stream_bits"] == g["stream_bits"]
    assert [f"{b:02X}" for b in s["stream"][:2]] == g["stream_bytes_hex"]
    assert s["groups"].tolist() == g["segments"]
    assert s["lane_off"][0, 0] == g["lane_off_first"] and (s["lane_off"][0, 1:] == g["lane_off_rest"]).all()
    assert s["sm"].size == 0
    out, rep = oracle_lib.decode_u8(blob, with_report=True)
    assert np.array_equal(out, c) and rep["entropy_bits"] == g["entropy_bits"]


@pytest.mark.parametrize("shuffle", [False, True])
def test_u8_all_byte_values_closed_form(oracle_lib, shuffle):
    c = (np.arange(65536) % 256).astype(np.uint8)
    if shuffle:
        c = np.random.default_rng(11).permutation(c)
    blob = oracle_lib.encode_lanes_u8(c)
    s = sections(blob)
    assert (s["code_len"] == 8).all()
    seg = min(4096, (15872 // (8 * 128)) * 128)                 # 1920 elements of 8 bits
    firsts = list(range(0, 65536, seg)) + [65536]
    assert s["groups"][:, 0].tolist() == firsts
    expect = np.concatenate([c[a:b][lane_permutation(b - a)] for a, b in zip(firsts[:-1], firsts[1:])])
    assert np.array_equal(s["stream"][:65536], expect)
    assert np.array_equal(oracle_lib.decode_u8(blob), c)


@pytest.mark.parametrize("A,M,B", [(128, 4096, 15872), (8, 512, 500)])
def test_u8_equals_bf16_kind_on_exponent_only_words(oracle_lib, A, M, B):
    from lossless_entropy_coded_amd.synth import make_code_workload
    wl = make_code_workload("int4_codes_8b", scale_rows=16)
    c = wl.codes
    u8 = sections(oracle_lib.encode_lanes_u8(c, group_align=A, group_max_elems=M, seg_max_bits=B))
    bf = sections(oracle_lib.encode_lanes(c.astype(np.uint16) << 7, group_align=A, group_max_elems=M,
                                          seg_max_bits=B))
    assert u8["elem_kind"] == 1 and bf["elem_kind"] == 0
    for key in ("code_len", "groups", "lane_off", "stream"):
        assert np.array_equal(u8[key], bf[key]), key
    assert u8["stream_bits"] == bf["stream_bits"] and u8["sm"].size == 0


def _rounded_gaussian_probs(bits, sigma):
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    Phi = lambda x: 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))
    p = []
    for k in range(lo, hi + 1):
        a = -math.inf if k == lo else (k - 0.5) / sigma
        b = math.inf if k == hi else (k + 0.5) / sigma
        p.append((Phi(b) if b != math.inf else 1.0) - (Phi(a) if a != -math.inf else 0.0))
    return np.array(p)


@pytest.mark.parametrize("bits,sigma", [(4, 1.5), (8, 20.0)])
def test_code_generator_closed_form(bits, sigma):
    """The stand-in codes follow round(N(0, sigma)) clipped (chi-squared test
    against the closed form; bins with fewer than 20 expected merged)."""
    from scipy.stats import chi2
    from lossless_entropy_coded_amd.synth import quantized_codes
    n = 400_000
    q = quantized_codes(np.random.default_rng(123), n, bits, sigma).astype(np.int64)
    p = _rounded_gaussian_probs(bits, sigma)
    obs = np.bincount(q, minlength=1 << bits).astype(np.float64)
    exp = p * n
    keep = exp >= 20
    obs_m = np.append(obs[keep], obs[~keep].sum())
    exp_m = np.append(exp[keep], exp[~keep].sum())
    if exp_m[-1] == 0:
        obs_m, exp_m = obs_m[:-1], exp_m[:-1]
    stat = ((obs_m - exp_m) ** 2 / exp_m).sum()
    assert stat < chi2.ppf(0.999, obs_m.size - 1)


@pytest.mark.parametrize("name", ["int8_codes_8b", "int4_codes_8b"])
def test_u8_round_trip_and_entropy_bound(oracle_lib, name):
    from lossless_entropy_coded_amd.synth import make_code_workload
    wl = make_code_workload(name, scale_rows=32)
    blob = oracle_lib.encode_lanes_u8(wl.codes, numels=wl.numels)
    out, rep = oracle_lib.decode_u8(blob, with_report=True)
    assert np.array_equal(out, wl.codes)
    assert rep["entropy_bits"] <= rep["mean_code_bits"] < rep["entropy_bits"] + 1
    # independent int4 pairs: the byte entropy is twice the code entropy
    p = _rounded_gaussian_probs(wl.bits, wl.sigma)
    H = -(p[p > 0] * np.log2(p[p > 0])).sum() * (2 if wl.bits == 4 else 1)
    assert abs(rep["entropy_bits"] - H) < 0.02


def test_u8_kind_checks(oracle_lib):
    c = np.arange(1000, dtype=np.uint16).astype(np.uint8)
    blob = oracle_lib.encode_lanes_u8(c)
    with pytest.raises(oracle_lib.OracleError) as ei:
        oracle_lib.decode(blob)
    assert ei.value.code == -15
    w = np.arange(1000, dtype=np.uint16)
    with pytest.raises(oracle_lib.OracleError) as ei:
        oracle_lib.decode_u8(oracle_lib.encode_lanes(w))
    assert ei.value.code == -15
    bad = blob.copy()
    bad[124] = 2
    assert oracle_lib.decode_status(bad) == -2
    chunked = oracle_lib.encode(w)
    chunked[124] = 1                        # version 2 has no element kind
    assert oracle_lib.decode_status(chunked) == -2
