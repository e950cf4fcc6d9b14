"""A seeded sweep over encoder options: for random combinations of layout,
coder, element kind, gap width, block size A, element cap M, segment bit cap
B, chunks per group G, thread count and input (length, distribution), the
product's writer and the oracle's writer give the same container byte for
byte, and the oracle decodes it to the input.  Where the options leave the
range the GPU decoder takes (A not a positive multiple of 8, M above 4096, a
lanes segment above 15872 bits) the product's writer refuses them with
WC_ERR_INVALID_ARG, and the oracle's container still decodes on the CPU."""
import numpy as np
import pytest


def _input(rng, n, kind):
    dist = rng.integers(0, 4)
    if kind == "u8":
        if dist == 0:
            return rng.integers(0, 256, n).astype(np.uint8)
        if dist == 1:
            return np.full(n, rng.integers(0, 256), np.uint8)
        sigma = float(rng.choice([0.7, 3.0, 20.0]))
        return (128 + np.clip(np.rint(rng.standard_normal(n) * sigma), -128, 127)).astype(np.uint8)
    if dist == 0:
        return rng.integers(0, 65536, n).astype(np.uint16)
    if dist == 1:
        return np.full(n, 0x3F80, np.uint16)
    sigma = float(rng.choice([1e-3, 0.02, 3.0]))
    x = (rng.standard_normal(n).astype(np.float32) * np.float32(sigma)).view(np.uint32)
    w = ((x + 0x7FFF + ((x >> 16) & 1)) >> 16).astype(np.uint16)
    if dist == 3:                                   # a sprinkle of special values
        special = np.array([0x0000, 0x8000, 0x0001, 0x7F80, 0xFF80, 0x7FC1], np.uint16)
        k = max(1, n // 50)
        w[rng.integers(0, n, k)] = special[rng.integers(0, special.size, k)]
    return w


CASES = list(range(160))


@pytest.fixture(scope="module")
def wc_lib():
    from lossless_entropy_coded_amd import wc
    return wc


def product_range(A, M, B=None):
    """Whether the product's writer takes these options (the GPU decoder's range)."""
    return A >= 8 and A % 8 == 0 and M <= 4096 and (B is None or B <= 15872)


def _product(wc, in_range, write):
    """The product writer's container, or None after checking that it refuses
    options outside its range."""
    if in_range:
        return write()
    with pytest.raises(wc.WCError) as ei:
        write()
    assert ei.value.status == wc.WC_ERR_INVALID_ARG
    return None


def build_case(wc, oracle_lib, case):
    """Case `case` of the sweep: (product container or None when the product's
    writer refuses the options, oracle container, input, element kind,
    description)."""
    rng = np.random.default_rng(1000 + case)
    variant = ["lanes-huffman", "lanes-rans", "chunks", "chunks-gap5"][case % 4]
    kind = "u8" if (variant.startswith("lanes") and rng.integers(0, 3) == 0) else "bf16"
    n = int(rng.choice([0, 1, 7, 8, 9, 63, 64, 65, 511, 4096, 4097, 20_000, 70_001]))
    parts = np.sort(rng.integers(0, n + 1, int(rng.integers(0, 4))))
    data = _input(rng, n, kind)
    tensors = np.split(data, parts)
    numels = [t.size for t in tensors]
    A = int(rng.choice([1, 8, 64, 120, 128])) if variant.startswith("chunks") else int(rng.choice([8, 64, 120, 128]))
    M = A * int(rng.integers(1, max(2, 4096 // A) + 1))
    threads = int(rng.choice([1, 2, 5]))
    desc = f"{variant} {kind} n={n} A={A} M={M}"
    if variant.startswith("chunks"):
        L = int(rng.choice([12, 16, 24]))
        G = int(rng.choice([64, 128, 256, 1000]))
        if A * L + 63 > 64 * G:
            G = -(-(A * L + 63) // 64)
        gap = 5 if variant.endswith("gap5") else 8
        a = _product(wc, product_range(A, M), lambda: wc.encode_host(
            tensors, layout="chunks", max_code_len=L, chunks_per_group=G, group_align=A, group_max_elems=M,
            gap_bits=gap, n_threads=threads))
        b = oracle_lib.encode(data, numels=numels, max_code_len=L, chunks_per_group=G, group_align=A,
                              group_max_elems=M, gap_bits=gap)
        desc += f" L={L} G={G} gap={gap}"
    elif variant == "lanes-rans":
        B = max(int(rng.choice([2048, 4096, 15872, 65535])), 2048 + (97 * A + 7) // 8)
        if kind == "u8":
            a = _product(wc, product_range(A, M, B), lambda: wc.encode_u8_host(
                tensors, coder="rans", group_align=A, group_max_elems=M, seg_max_bits=B, n_threads=threads))
            b = oracle_lib.encode_lanes_rans_u8(data, numels=numels, group_align=A, group_max_elems=M, seg_max_bits=B)
        else:
            a = _product(wc, product_range(A, M, B), lambda: wc.encode_host(
                tensors, coder="rans", group_align=A, group_max_elems=M, seg_max_bits=B, n_threads=threads))
            b = oracle_lib.encode_lanes_rans(data, numels=numels, group_align=A, group_max_elems=M, seg_max_bits=B)
        desc += f" B={B}"
    else:
        L = int(rng.choice([11, 16, 24]))
        B = max(int(rng.choice([500, 4096, 15872, 65535])), A * L)
        if kind == "u8":
            a = _product(wc, product_range(A, M, B), lambda: wc.encode_u8_host(
                tensors, max_code_len=L, group_align=A, group_max_elems=M, seg_max_bits=B, n_threads=threads))
            b = oracle_lib.encode_lanes_u8(data, numels=numels, max_code_len=L, group_align=A, group_max_elems=M,
                                           seg_max_bits=B)
        else:
            a = _product(wc, product_range(A, M, B), lambda: wc.encode_host(
                tensors, max_code_len=L, group_align=A, group_max_elems=M, seg_max_bits=B, n_threads=threads))
            b = oracle_lib.encode_lanes(data, numels=numels, max_code_len=L, group_align=A, group_max_elems=M,
                                        seg_max_bits=B)
        desc += f" L={L} B={B}"
    return a, b, data, kind, desc


@pytest.mark.parametrize("case", CASES)
def test_product_writer_equals_oracle_writer(wc_lib, oracle_lib, case):
    a, b, data, kind, desc = build_case(wc_lib, oracle_lib, case)
    assert a is None or np.array_equal(a, b), desc
    out = oracle_lib.decode_u8(b) if kind == "u8" else oracle_lib.decode(b)
    assert np.array_equal(out, data), desc


def test_sweep_covers_both_sides_of_the_range(wc_lib, oracle_lib):
    """The sweep holds options the product writes and options it refuses."""
    written = sum(build_case(wc_lib, oracle_lib, c)[0] is not None for c in CASES[:48])
    assert 0 < written < 48
