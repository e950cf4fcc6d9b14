"""GPU parity of the symbol-plane decode (u8-kind interleaved-lane
containers: planes of 8-bit quantized codes), called through the C ABI,
against the CPU oracle and the identity, bit-exact.  Outputs are framed by
canary guard bands that must survive every decode."""
import numpy as np
import pytest

from gpu_util import log, to_device_aligned

pytestmark = pytest.mark.gpu

CANARY = 0xA5
GUARD = 512


@pytest.fixture(scope="module")
def wc():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from lossless_entropy_coded_amd import wc as mod
    return mod


def gpu_decode_u8(wc, blob, stream=None):
    import torch
    with wc.Plan(blob) as plan:
        assert plan.format()[:2] == (3, 1)
        _, dblob = to_device_aligned(blob)
        buf = torch.full((plan.n_elems + 2 * GUARD,), CANARY, dtype=torch.uint8, device="cuda")
        out = buf[GUARD:GUARD + plan.n_elems]
        wc.decode_u8_async(plan, dblob, out, stream=stream)
        torch.cuda.synchronize()
        assert bool((buf[:GUARD] == CANARY).all()) and bool((buf[GUARD + plan.n_elems:] == CANARY).all()), \
            "decode wrote outside its output range"
        return out.cpu().numpy()


def test_u8_worked_example(wc):
    c = np.array([5, 3, 5, 7, 5, 9, 3, 5], np.uint8)
    log("case: u8 worked example")
    assert np.array_equal(gpu_decode_u8(wc, wc.encode_u8_host([c])), c)


@pytest.mark.parametrize("shuffle", [False, True])
def test_u8_all_byte_values(wc, oracle_lib, shuffle):
    c = (np.arange(65536) % 256).astype(np.uint8)
    if shuffle:
        c = np.random.default_rng(5).permutation(c)
    for writer in ("product", "oracle"):
        blob = wc.encode_u8_host([c]) if writer == "product" else oracle_lib.encode_lanes_u8(c)
        log(f"case: u8 all byte values shuffle={shuffle} writer={writer}")
        assert np.array_equal(gpu_decode_u8(wc, blob), c)


def test_u8_tiny_and_skewed(wc, oracle_lib):
    rng = np.random.default_rng(77)
    cases = [np.array([200], np.uint8)]
    for n in list(range(1, 40)) + [63, 64, 65, 511, 512, 513, 4095, 4096, 4097, 8200]:
        cases.append(rng.integers(0, 256, n).astype(np.uint8))
        cases.append(np.full(n, 128, np.uint8))
        cases.append((128 + np.clip(np.rint(rng.standard_normal(n) * 3), -128, 127)).astype(np.uint8))
    for i, c in enumerate(cases):
        log(f"case: u8 tiny #{i} n={c.size}")
        blob = wc.encode_u8_host([c]) if i % 2 == 0 else oracle_lib.encode_lanes_u8(c)
        assert np.array_equal(gpu_decode_u8(wc, blob), c), f"case {i}"


@pytest.mark.parametrize("A,M,B", [(8, 4096, 15872), (64, 1024, 4096), (8, 512, 500), (256, 4096, 8192)])
def test_u8_segment_shapes(wc, oracle_lib, A, M, B):
    from lossless_entropy_coded_amd.synth import make_code_workload
    wl = make_code_workload("int8_codes_8b", scale_rows=96)
    for writer in ("product", "oracle"):
        blob = (wc.encode_u8_host(wl.tensors(), group_align=A, group_max_elems=M, seg_max_bits=B)
                if writer == "product" else
                oracle_lib.encode_lanes_u8(wl.codes, numels=wl.numels, group_align=A, group_max_elems=M,
                                           seg_max_bits=B))
        log(f"case: u8 A={A} M={M} B={B} writer={writer}")
        assert np.array_equal(gpu_decode_u8(wc, blob), wl.codes)


@pytest.mark.parametrize("name,first_code_table", [
    ("int8_codes_8b", "1"), ("int4_codes_8b", "1"), ("int4_codes_8b", "0")])
def test_u8_workload_full_size(wc, oracle_lib, monkeypatch, name, first_code_table):
    """The full 8B-shape code planes (218 M int8 codes; 109 M bytes of int4
    pairs), one launch each, against the input and the oracle; int4 pairs
    also on the wide table (WC_FIRST_CODE_TABLE=0)."""
    from lossless_entropy_coded_amd.synth import make_code_workload
    monkeypatch.setenv("WC_FIRST_CODE_TABLE", first_code_table)
    wl = make_code_workload(name)
    blob = wc.encode_u8_host(wl.tensors())
    log(f"case: u8 full {name} first_code_table={first_code_table} n={wl.n} container={blob.size}")
    with wc.Plan(blob) as plan:
        # code planes: one launch of 8-wave workgroups, whatever the size
        shape = plan.decode_shape()
        assert shape["launches"] == 1 and shape["waves_per_group"] == 8
        assert shape["grid"] == plan.stats()["grid"]
    got = gpu_decode_u8(wc, blob)
    assert np.array_equal(got, wl.codes)
    if first_code_table == "1":
        log(f"case: u8 full {name} oracle decode")
        assert np.array_equal(got, oracle_lib.decode_u8(blob))


def one_code_expected(lens, kd):
    """The planner's rule for code planes: one code per lookup when no code
    exceeds 16 bits and either the shortest is longer than half the table
    index (no table entry holds two) or every code fits the index (the
    first-code table replaces the multi-codeword table)."""
    present = lens[lens > 0]
    shortest, longest = int(present.min()), int(present.max())
    return longest <= 16 and (2 * shortest > kd or (present.size >= 2 and longest <= kd))


@pytest.mark.parametrize("sigma,max_len,one_code,longest_over", [
    (20.0, 0, True, False),     # shortest code 6 bits, none longer than the 11-bit index
    (40.0, 24, True, True),     # shortest 6, longest 14: the long-code path inside one-code lookups
    (30.0, 24, False, True),    # shortest 6, longest 18: four codes may not fit 64 bits
    (20.0, 24, False, True),    # shortest 5 and codes past the index: the wide table
    (3.0, 0, True, False),      # shortest 3, none past the index: the first-code table
])
def test_u8_one_code_lookups(wc, oracle_lib, sigma, max_len, one_code, longest_over):
    """Code planes take one code per lookup when no code is longer than 16
    bits and either no table entry can hold two codes (shortest code longer
    than half the 11-bit index) or every code fits the index (a table of
    each window's first code): eight codes per 96-bit window when none is
    longer than the index, else four per 64-bit window.  The others take
    the wide table.  All are bit-exact against the input and the oracle."""
    from container_view import sections
    from lossless_entropy_coded_amd.synth import quantized_codes
    rng = np.random.default_rng(int(sigma * 10) + max_len)
    c = quantized_codes(rng, 300_000, 8, sigma)
    blob = wc.encode_u8_host([c], max_code_len=max_len)
    lens = sections(blob)["code_len"]
    with wc.Plan(blob) as plan:
        kd = plan.stats()["decode_bits"]
    assert one_code_expected(lens, kd) == one_code
    assert (int(lens.max()) > kd) == longest_over
    log(f"case: u8 one-code sigma={sigma} max_len={max_len} one_code={one_code}")
    got = gpu_decode_u8(wc, blob)
    assert np.array_equal(got, c)
    assert np.array_equal(got, oracle_lib.decode_u8(blob))


@pytest.mark.parametrize("sigma,max_len,first_code_table,one_code", [
    (20.0, 10, "1", True),      # shortest code longer than 5 bits
    (3.0, 10, "1", True),       # shortest 3: the first-code table
    (3.0, 10, "0", False),      # the same plane on the wide table (11-bit index)
])
def test_u8_ten_bit_index(wc, oracle_lib, monkeypatch, sigma, max_len, first_code_table, one_code):
    """With a 10-bit table index (WC_DECODE_BITS=10) and no code longer than
    it: int8-like and int4-like planes take the one-code path with eight codes
    (at most 80 bits) per 96-bit window; with WC_FIRST_CODE_TABLE=0 int4-like
    planes take the wide table (11-bit index) in two phases.  Bit-exact
    against the input and the oracle."""
    from container_view import sections
    from lossless_entropy_coded_amd.synth import quantized_codes
    monkeypatch.setenv("WC_DECODE_BITS", "10")
    monkeypatch.setenv("WC_FIRST_CODE_TABLE", first_code_table)
    rng = np.random.default_rng(int(sigma * 100) + max_len)
    c = quantized_codes(rng, 250_000, 8, sigma)
    blob = wc.encode_u8_host([c], max_code_len=max_len)
    lens = sections(blob)["code_len"]
    with wc.Plan(blob) as plan:
        assert plan.stats()["decode_bits"] == 10
    assert int(lens.max()) <= 10 and (2 * int(lens[lens > 0].min()) > 10 or first_code_table == "1") == one_code
    log(f"case: u8 ten-bit index sigma={sigma} first_code_table={first_code_table} one_code={one_code}")
    got = gpu_decode_u8(wc, blob)
    assert np.array_equal(got, c)
    assert np.array_equal(got, oracle_lib.decode_u8(blob))


@pytest.mark.parametrize("sigma,first_code_table", [(3.0, "1"), (3.0, "0"), (20.0, "1")])
def test_u8_small_segments_every_tail(wc, oracle_lib, monkeypatch, sigma, first_code_table):
    """Single-segment containers of 8 * full + r codes for every tail length
    r and full blocks on either side of each lane and phase boundary: the
    lanes after the one holding the partial last block have fewer symbols
    (none in the wide table's second phase), and nothing they do may touch
    the partial block's bytes.  int4-like planes run on the first-code table
    and, with WC_FIRST_CODE_TABLE=0, on the wide table."""
    from lossless_entropy_coded_amd.synth import quantized_codes
    monkeypatch.setenv("WC_FIRST_CODE_TABLE", first_code_table)
    rng = np.random.default_rng(int(sigma) + 77)
    fulls = [0, 1, 5, 36, 63, 64, 65, 100, 127, 200, 255, 256, 257, 300, 447, 510]
    log(f"case: u8 small segments sigma={sigma} first_code_table={first_code_table}: "
        f"n = 8 * full + r, full in {fulls}, r in 0..7")
    for full in fulls:
        for r in range(8):
            n = 8 * full + r
            if n == 0:
                continue
            c = quantized_codes(rng, n, 8, sigma)
            blob = wc.encode_u8_host([c])
            got = gpu_decode_u8(wc, blob)
            assert np.array_equal(got, c), f"n = {n} (full {full}, tail {r}), sigma {sigma}"
    assert np.array_equal(oracle_lib.decode_u8(blob), c)


@pytest.mark.parametrize("name", ["int8_codes_8b", "int4_codes_8b"])
def test_u8_corrupted_stream_stays_in_bounds(wc, name):
    from container_view import sections
    from lossless_entropy_coded_amd.synth import make_code_workload
    wl = make_code_workload(name, scale_rows=128)
    blob = wc.encode_u8_host(wl.tensors())
    s = sections(blob)
    rng = np.random.default_rng(9)
    for k in (1, 100, 5000):
        b = blob.copy()
        pos = rng.integers(0, s["stream_bits"], size=k)
        np.bitwise_xor.at(b, s["off_stream"] + pos // 8, (0x80 >> (pos % 8)).astype(np.uint8))
        log(f"case: u8 corrupted flips={k}")
        assert gpu_decode_u8(wc, b).size == wl.n


def test_u8_single_symbol_corrupted_stream_ends(wc):
    """A one-symbol code plane has the incomplete code "0": windows that start
    with a 1 bit match no code, so the planner keeps the long-code lookup
    (which always advances) in its loop.  A stream corrupted to 1 bits still
    ends and writes nothing outside the output; the valid stream decodes
    exactly."""
    from container_view import sections
    c = np.full(100_003, 77, np.uint8)
    blob = wc.encode_u8_host([c])
    log("case: u8 one symbol, valid")
    assert np.array_equal(gpu_decode_u8(wc, blob), c)
    s = sections(blob)
    nbytes = (s["stream_bits"] + 7) // 8
    for fill in (0xFF, 0xA5):
        b = blob.copy()
        b[s["off_stream"]:s["off_stream"] + nbytes - 1] = fill
        log(f"case: u8 one symbol, stream bytes set to {fill:#x}")
        assert gpu_decode_u8(wc, b).size == c.size


def test_u8_kind_checks(wc):
    import torch
    c = np.arange(4096).astype(np.uint8)
    w = np.arange(4096, dtype=np.uint16)
    with wc.Plan(wc.encode_u8_host([c])) as plan:
        out = torch.zeros(4096, dtype=torch.int16, device="cuda")
        with pytest.raises(wc.WCError) as ei:
            wc.decode_async(plan, out, out)
        assert ei.value.status == wc.WC_ERR_INVALID_ARG
    with wc.Plan(wc.encode_host([w])) as plan:
        assert plan.format() == (3, 0, 0)
        out = torch.zeros(8192, dtype=torch.uint8, device="cuda")
        with pytest.raises(wc.WCError) as ei:
            wc.decode_u8_async(plan, out, out)
        assert ei.value.status == wc.WC_ERR_INVALID_ARG
