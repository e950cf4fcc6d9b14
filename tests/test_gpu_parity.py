"""GPU parity: the gfx950 decode kernel, called through the C ABI, against the
CPU oracle and against the identity (decode(encode(W)) == W), bit-exact.

Every output buffer is framed by canary guard bands that must survive every
decode.  Expected values come only from the seeded generators, the oracle or
closed forms, never from the GPU.
"""
import os

import numpy as np
import pytest

from gpu_util import GuardedOutput, gpu_decode, log, to_device_aligned

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


def test_worked_example(wc):
    w = np.array([0x3C80, 0x3C00, 0x3C80, 0x3B80, 0x3C80, 0x3D00, 0x3C00, 0x3C80], np.uint16)
    log("case: worked example n=8")
    assert np.array_equal(gpu_decode(wc, wc.encode_host([w], layout="chunks")), w)


@pytest.mark.parametrize("shuffle", [False, True])
def test_all_bf16_patterns(wc, oracle_lib, shuffle):
    w = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if shuffle:
        w = np.random.default_rng(99).permutation(w)
    for writer in ("product", "oracle"):
        blob = wc.encode_host([w], layout="chunks") if writer == "product" else oracle_lib.encode(w, chunks_per_group=wc.GROUP_CHUNKS)
        log(f"case: all 65536 patterns shuffle={shuffle} writer={writer}")
        assert np.array_equal(gpu_decode(wc, blob), w)


def test_tiny_and_special_sequences(wc, oracle_lib):
    rng = np.random.default_rng(2024)
    special = np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x7F80, 0xFF80, 0x7FC1, 0xFFFF, 0x3F80, 0xBF80],
                       np.uint16)
    cases = [np.zeros(0, np.uint16), np.array([0x1234], np.uint16)]
    for n in list(range(1, 40)) + [63, 64, 65, 127, 128, 129, 255, 256, 257, 1000, 4095, 4096, 4097]:
        cases.append(special[rng.integers(0, special.size, size=n)])
        cases.append(rng.integers(0, 65536, size=n, dtype=np.uint16))
        cases.append(np.full(n, 0x3C00, np.uint16))
    for i, w in enumerate(cases):
        log(f"case: tiny #{i} n={w.size}")
        blob = wc.encode_host([w], layout="chunks") if i % 2 == 0 else oracle_lib.encode(w, chunks_per_group=wc.GROUP_CHUNKS)
        got = gpu_decode(wc, blob)
        assert np.array_equal(got, w), f"case {i} n={w.size}"


def _fib_alphabet(prefix):
    fib = [1, 1]
    while len(fib) < 25:
        fib.append(fib[-1] + fib[-2])
    counts = dict(zip(range(100, 125), [16 * f for f in fib[::-1]]))   # x16 keeps the same code tree
    seq = list(prefix)
    for s in seq:
        counts[s] -= 1
    rng = np.random.default_rng(len(seq))
    rest = np.concatenate([np.full(c, s, np.uint16) for s, c in counts.items()])
    seq = np.concatenate([np.array(seq, np.uint16), rng.permutation(rest)])
    return (seq << 7).astype(np.uint16) | rng.integers(0, 128, size=seq.size, dtype=np.uint16)


@pytest.mark.parametrize("prefix", [[100] * 63 + [124], [100] * 64, [124] * 10, [123, 124] * 8, []])
def test_long_codes_and_chunk_boundaries(wc, oracle_lib, prefix):
    """Code lengths up to 24 bits (the long-code path), codewords straddling
    chunk boundaries by up to 23 bits, both writers."""
    w = _fib_alphabet(prefix)
    for writer in ("product", "oracle"):
        blob = wc.encode_host([w], layout="chunks") if writer == "product" else oracle_lib.encode(w, chunks_per_group=wc.GROUP_CHUNKS)
        log(f"case: fib alphabet prefix_len={len(prefix)} writer={writer} n={w.size}")
        assert np.array_equal(gpu_decode(wc, blob), w)


def _many_rare_exponents(n=400_000, n_rare=200, seed=7):
    """Eight exponents with counts n/2, n/4, ..., n/256 take code lengths 1..8;
    200 rare exponents share the remaining 1/256 of the elements, so their
    codes are about 15-16 bits long and spread over several 10- and 11-bit
    code prefixes (more than a second-level table of three prefixes covers)."""
    rng = np.random.default_rng(seed)
    head = [120, 119, 121, 118, 122, 117, 123, 116]
    rare = np.array([e for e in range(256) if e not in head][:n_rare], np.uint16)
    parts = []
    left = n
    for i, e in enumerate(head):
        k = n >> (i + 1)
        parts.append(np.full(k, e, np.uint16))
        left -= k
    parts.append(rare[np.arange(left) % n_rare])
    exps = rng.permutation(np.concatenate(parts))
    sm = rng.integers(0, 256, n).astype(np.uint16)
    return (((sm & 0x80) << 8) | (exps << 7) | (sm & 0x7F)).astype(np.uint16)


@pytest.mark.parametrize("bits", [(12, 11), (12, 10), (11, 11), (11, 10), (10, 10)])
def test_many_long_code_prefixes(wc, oracle_lib, env_knob, bits):
    """Long codes of many distinct prefixes, at every table width: some resolve
    in one second-level lookup, others need the length-by-length search."""
    w = _many_rare_exponents()
    blob = wc.encode_host([w], layout="chunks")
    env_knob("WC_COUNT_BITS", bits[0])
    env_knob("WC_DECODE_BITS", bits[1])
    log(f"case: many rare exponents n={w.size} table bits={bits}")
    with wc.Plan(blob) as plan:
        assert (plan.stats()["count_bits"], plan.stats()["decode_bits"]) == bits
        assert np.array_equal(gpu_decode(wc, blob, plan=plan), w)


@pytest.mark.parametrize("bits", [(12, 11), (12, 10), (11, 11), (11, 10), (10, 10)])
@pytest.mark.parametrize("grid", [1, 7, 16, 0])
@pytest.mark.parametrize("waves", [4, 8])
def test_table_width_and_grid_invariance(wc, env_knob, bits, grid, waves):
    """Every table width, wavefronts per workgroup and grid size (one
    workgroup looping over every group; grids that are and are not a multiple
    of the die count) decodes the same bits."""
    from lossless_entropy_coded_amd.synth import make_workload
    wl = make_workload("heavy_tail_14k", scale_rows=512)
    blob = wc.encode_host(wl.tensors(), layout="chunks")
    env_knob("WC_COUNT_BITS", bits[0])
    env_knob("WC_DECODE_BITS", bits[1])
    env_knob("WC_GRID", grid or None)
    env_knob("WC_WAVES", waves)
    log(f"case: heavy_tail rows=512 table bits={bits} grid={grid} waves={waves}")
    with wc.Plan(blob) as plan:
        st = plan.stats()
        assert (st["count_bits"], st["decode_bits"]) == bits
        if grid:
            assert st["grid"] == grid
        assert np.array_equal(gpu_decode(wc, blob, plan=plan), wl.bits)


@pytest.mark.parametrize("name", ["matrix_1k", "attn_4k_zeros", "block_8b", "heavy_tail_14k", "block_70b"])
def test_workload_full_size(wc, oracle_lib, name):
    """Full-size workloads, one launch each, in the benchmark's launch configuration."""
    import torch
    from lossless_entropy_coded_amd.synth import make_workload
    wl = make_workload(name)
    blob = wc.encode_host(wl.tensors(), layout="chunks")
    log(f"case: full {name} n={wl.n} container={blob.size}")
    with wc.Plan(blob) as plan:
        assert plan.n_elems == wl.n and plan.tensor_numels == wl.numels
        _, dblob = to_device_aligned(blob)
        out = GuardedOutput(wl.n)
        wc.decode_async(plan, dblob, out.out)
        torch.cuda.synchronize()
        assert out.guards_intact()
        ref = torch.from_numpy(wl.bits.view(np.int16)).cuda()
        assert torch.equal(out.out, ref), "GPU decode differs from the input weights"
        # every tensor view sits at its table offset
        for off, k in zip(plan.tensor_offsets, plan.tensor_numels):
            assert torch.equal(out.out[off:off + k], ref[off:off + k])
        del ref
        if wl.n <= 300_000_000:
            got = out.host()
            log(f"case: full {name} oracle decode")
            assert np.array_equal(got, oracle_lib.decode(blob))


@pytest.mark.parametrize("name,rows", [("matrix_1k", None), ("block_8b", 256), ("heavy_tail_14k", 2048)])
def test_oracle_written_containers(wc, oracle_lib, name, rows):
    """Containers written by the oracle's own serial writer decode exactly."""
    from lossless_entropy_coded_amd.synth import make_workload
    wl = make_workload(name, scale_rows=rows)
    blob = oracle_lib.encode(wl.bits, numels=wl.numels, chunks_per_group=wc.GROUP_CHUNKS)
    log(f"case: oracle-written {name} rows={rows}")
    assert np.array_equal(gpu_decode(wc, blob), wl.bits)


@pytest.mark.parametrize("align", [8, 64, 120, 128, 256])
@pytest.mark.parametrize("writer", ["product", "oracle"])
def test_group_block_sizes(wc, oracle_lib, align, writer):
    """Any block size that is a multiple of 8 decodes exactly: groups then
    start anywhere on an 8-element boundary, not only on cache lines."""
    from lossless_entropy_coded_amd.synth import make_workload
    wl = make_workload("heavy_tail_14k", scale_rows=256)
    M = wc.GROUP_MAX_ELEMS // align * align            # the largest multiple of A the decoder accepts
    if writer == "product":
        blob = wc.encode_host(wl.tensors(), group_align=align, group_max_elems=M, layout="chunks")
    else:
        blob = oracle_lib.encode(wl.bits, numels=wl.numels, chunks_per_group=wc.GROUP_CHUNKS, group_align=align,
                                 group_max_elems=M)
    log(f"case: group_align={align} writer={writer}")
    assert np.array_equal(gpu_decode(wc, blob), wl.bits)


@pytest.mark.parametrize("G", [49, 64, 256, 1000])
@pytest.mark.parametrize("writer", ["product", "oracle"])
@pytest.mark.parametrize("gap_bits", [8, 5])
def test_chunks_per_group(wc, oracle_lib, G, writer, gap_bits):
    """Any group width in chunks decodes exactly: a group whose codewords span
    more than 128 chunks is decoded in passes of 128 chunks.  High-entropy
    values (about 16-bit codes) make groups of 4096 elements span up to 1024
    chunks, i.e. up to eight passes; the low-entropy block keeps groups
    within one pass."""
    from lossless_entropy_coded_amd.synth import make_workload
    rng = np.random.default_rng(G)
    wide = rng.permutation(np.arange(65536, dtype=np.uint32).astype(np.uint16))[:50_000]
    wl = make_workload("heavy_tail_14k", scale_rows=128)
    for label, w, numels in (("all patterns", wide, None), ("heavy_tail_14k", wl.bits, wl.numels)):
        if writer == "product":
            parts = [w] if numels is None else wl.tensors()
            blob = wc.encode_host(parts, layout="chunks", chunks_per_group=G, gap_bits=gap_bits)
        else:
            blob = oracle_lib.encode(w, numels=numels, chunks_per_group=G, gap_bits=gap_bits)
        log(f"case: chunks_per_group={G} writer={writer} gap={gap_bits} {label}")
        assert np.array_equal(gpu_decode(wc, blob), w)


def test_corrupted_stream_stays_in_bounds(wc):
    """Valid metadata, garbage bit stream: output may be wrong, but nothing is
    written outside [out, out + n)."""
    from container_view import sections
    from lossless_entropy_coded_amd.synth import make_workload
    wl = make_workload("matrix_1k", scale_rows=256)
    blob = wc.encode_host(wl.tensors(), layout="chunks")
    s = sections(blob)
    rng = np.random.default_rng(3)
    nbytes = (s["stream_bits"] + 7) // 8
    variants = []
    for k in (1, 10, 1000):
        b = blob.copy()
        pos = rng.integers(0, s["stream_bits"], size=k)
        np.bitwise_xor.at(b, s["off_stream"] + pos // 8, (0x80 >> (pos % 8)).astype(np.uint8))
        variants.append(("flip%d" % k, b))
    b = blob.copy()
    b[s["off_stream"]:s["off_stream"] + nbytes - 1] = 0xFF
    variants.append(("ones", b))
    b = blob.copy()
    b[s["off_stream"]:s["off_stream"] + nbytes - 1] = 0x00
    variants.append(("zeros", b))
    # group bit offsets that pass wc_plan's checks but are not codeword starts
    for shift in (1, 23, 63):
        b = blob.copy()
        for g in range(1, int(s["n_groups"]), 3):
            at = s["off_gs"] + 16 * g + 8
            v = np.uint64(int(s["groups"][g, 1]) + shift)
            b[at:at + 8] = np.frombuffer(v.tobytes(), np.uint8)
        variants.append(("group-bits+%d" % shift, b))
    for tag, b in variants:
        log(f"case: corrupted stream {tag}")
        got = gpu_decode(wc, b)          # asserts the guard bands
        assert got.size == wl.n


def test_plan_reuse_across_streams_and_repeats(wc):
    import torch
    from lossless_entropy_coded_amd.synth import make_workload
    wl = make_workload("attn_4k_zeros", scale_rows=1024)
    blob = wc.encode_host(wl.tensors(), layout="chunks")
    ref = torch.from_numpy(wl.bits.view(np.int16)).cuda()
    log("case: two streams, repeated decodes")
    with wc.Plan(blob) as plan:
        _, dblob = to_device_aligned(blob)
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        outs = [GuardedOutput(wl.n) for _ in range(6)]
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            wc.decode_async(plan, dblob, o.out, stream=(s1 if i % 2 else s2))
        torch.cuda.synchronize()
        for o in outs:
            assert o.guards_intact() and torch.equal(o.out, ref)


def test_argument_checks(wc):
    import torch
    w = np.arange(4096, dtype=np.uint16)
    blob = wc.encode_host([w], layout="chunks")
    with wc.Plan(blob) as plan:
        _, dblob = to_device_aligned(blob)
        out = torch.empty(w.size + 16, dtype=torch.int16, device="cuda")
        log("case: misaligned output pointer")
        with pytest.raises(wc.WCError) as ei:
            wc.decode_async(plan, dblob, out.data_ptr() + 2)
        assert ei.value.status == wc.WC_ERR_INVALID_ARG
        with pytest.raises(wc.WCError) as ei:
            wc.decode_async(plan, dblob.data_ptr() + 16, out)
        assert ei.value.status == wc.WC_ERR_INVALID_ARG
        with pytest.raises(wc.WCError):
            wc.decode_async(plan, 0, out)
    empty = wc.encode_host([np.zeros(0, np.uint16)], layout="chunks")
    with wc.Plan(empty) as plan:
        assert plan.n_elems == 0
        assert plan.decode_shape()["launches"] == 0
        wc.decode_async(plan, 0, 0)       # n = 0 is a no-op
        torch.cuda.synchronize()


@pytest.mark.parametrize("rounds", [1, 2])
@pytest.mark.parametrize("layout,coder", [("lanes", "huffman"), ("lanes", "rans"), ("chunks", "huffman")])
def test_decode_in_several_launches(wc, env_knob, rounds, layout, coder):
    """A decode split into consecutive launches of `rounds` rounds of the
    persistent grid each (WC_LAUNCH_ROUNDS, read by wc_plan; large
    containers are split this way by default) is bit-exact: every launch
    starts at its own first segment."""
    from lossless_entropy_coded_amd.synth import make_workload
    wl = make_workload("heavy_tail_14k")              # 58.7 M elements: about 4.7 rounds
    blob = wc.encode_host(wl.tensors(), layout=layout, coder=coder)
    env_knob("WC_LAUNCH_ROUNDS", rounds)
    log(f"case: {layout} {coder} decode in launches of {rounds} rounds, n={wl.n}")
    with wc.Plan(blob) as plan:
        # wc_plan_decode_shape reports the split: ceil(rounds of the grid /
        # rounds per launch) launches of the plain decode's own shape
        shape, st = plan.decode_shape(), plan.stats()
        total = -(-st["n_groups"] // (shape["waves_per_group"] * shape["grid"]))
        assert shape["grid"] == st["grid"] and shape["waves_per_group"] == 4
        assert total >= 4 and shape["launches"] == -(-total // rounds), (shape, st)
    assert np.array_equal(gpu_decode(wc, blob), wl.bits)
