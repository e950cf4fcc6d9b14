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


@pytest.mark.parametrize("name", ["int8_codes_8b", "int4_codes_8b"])
def test_u8_workload_full_size(wc, oracle_lib, name):
    """The full 8B-shape code planes (218 M int8 codes; 109 M bytes of int4
    pairs), one launch each, against the input and the oracle."""
    from lossless_entropy_coded_amd.synth import make_code_workload
    wl = make_code_workload(name)
    blob = wc.encode_u8_host(wl.tensors())
    log(f"case: u8 full {name} n={wl.n} container={blob.size}")
    got = gpu_decode_u8(wc, blob)
    assert np.array_equal(got, wl.codes)
    log(f"case: u8 full {name} oracle decode")
    assert np.array_equal(got, oracle_lib.decode_u8(blob))


@pytest.mark.parametrize("sigma,max_len,one_code,longest_over", [
    (20.0, 0, True, False),     # shortest code 6 bits, none longer than the 11-bit index
    (40.0, 24, True, True),     # shortest 6, longest 14: the long-code path inside one-code lookups
    (30.0, 24, False, True),    # shortest 6, longest 18: four codes may not fit 64 bits
    (20.0, 24, False, True),    # shortest 5: two codes can share a lookup
    (3.0, 0, False, False),     # shortest 3: up to three codes per lookup
])
def test_u8_one_code_lookups(wc, oracle_lib, sigma, max_len, one_code, longest_over):
    """Code planes whose shortest code is longer than half the 11-bit table
    index never see two codes in one table entry; when no code is longer than
    16 bits the decoder takes one code per lookup, four per 64-bit window and
    per aligned word.  The others take the multi-code loop.  Both are
    bit-exact against the input and the oracle."""
    from container_view import sections
    from lossless_entropy_coded_amd.synth import quantized_codes
    rng = np.random.default_rng(int(sigma * 10) + max_len)
    c = quantized_codes(rng, 300_000, 8, sigma)
    blob = wc.encode_u8_host([c], max_code_len=max_len)
    lens = sections(blob)["code_len"]
    with wc.Plan(blob) as plan:
        kd = plan.stats()["decode_bits"]
    assert (2 * int(lens[lens > 0].min()) > kd and int(lens.max()) <= 16) == one_code
    assert (int(lens.max()) > kd) == longest_over
    log(f"case: u8 one-code sigma={sigma} max_len={max_len} one_code={one_code}")
    got = gpu_decode_u8(wc, blob)
    assert np.array_equal(got, c)
    assert np.array_equal(got, oracle_lib.decode_u8(blob))


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
