"""GPU tests of the debug status word (plans made with WC_DEBUG=1).

The chunks-layout kernels check, per group, that the codewords starting in
the group's bits number exactly its elements, and OR WC_DEBUG_GROUP_COUNT into
the plan's status word when they do not.  Valid containers must leave the
word clear; a stream whose bits are all zero must set it, which the test
proves from the container alone: the chunks of a group split its bits into
disjoint ranges that together cover them, and over zero bits every codeword
is the first canonical one (all zeros, the shortest length L), so a group of
n elements whose bit length exceeds L * n starts more than n codewords.
"""
import numpy as np
import pytest

from gpu_util import gpu_decode, log, to_device_aligned

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wc():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from lossless_entropy_coded_amd import wc as mod
    return mod


def _fused(wc, plan, dblob, shapes):
    """All matrices of the container in one fused call; returns host y arrays."""
    import torch
    from lossless_entropy_coded_amd.synth import gemv_input
    ops, ys = [], []
    for k, s in enumerate(shapes):
        if len(s) != 2:
            continue
        x = torch.from_numpy(gemv_input(s[1]).view(np.int16)).cuda()
        y = torch.empty(s[0], dtype=torch.float32, device="cuda")
        ops.append((k, s[1], x, y))
        ys.append(y)
    need = wc.decode_gemv_work_bytes(plan, ops)
    work = torch.empty(need // 4 + 64, dtype=torch.float32, device="cuda")
    wc.decode_gemv_async(plan, dblob, ops, work, need)
    torch.cuda.synchronize()
    return [y.cpu().numpy() for y in ys]


def _zero_stream(blob):
    """The container with every stream byte but the last set to zero, and
    the first group whose bits lie in those bytes and exceed L * n."""
    from container_view import sections
    s = sections(blob)
    lens = s["code_len"].astype(np.int64)
    L = int(lens[lens > 0].min())
    nbytes = (int(s["stream_bits"]) + 7) // 8
    b = blob.copy()
    b[s["off_stream"]:s["off_stream"] + nbytes - 1] = 0
    g = s["groups"].astype(np.int64)
    over = [k for k in range(int(s["n_groups"]))
            if g[k + 1, 1] <= 8 * (nbytes - 1) and g[k + 1, 1] - g[k, 1] > L * (g[k + 1, 0] - g[k, 0])]
    return b, over


def test_plan_without_debug_refuses(wc, monkeypatch):
    monkeypatch.delenv("WC_DEBUG", raising=False)
    blob = wc.encode_host([np.arange(4096, dtype=np.uint16)], layout="chunks")
    log("case: debug status of a plan made without WC_DEBUG")
    with wc.Plan(blob) as plan:
        with pytest.raises(wc.WCError) as ei:
            wc.plan_debug_status(plan)
        assert ei.value.status == wc.WC_ERR_INVALID_ARG


@pytest.mark.parametrize("enc", [dict(layout="chunks"), dict(layout="chunks", chunks_per_group=1000),
                                 dict(layout="chunks", gap_bits=5), dict(layout="lanes"),
                                 dict(layout="lanes", coder="rans")],
                         ids=["chunks", "chunks_g1000", "chunks5", "lanes", "rans"])
def test_valid_containers_leave_word_clear(wc, oracle_lib, monkeypatch, enc):
    """Decode and fused product of valid containers: bit-exact output, and
    the status word stays 0."""
    from lossless_entropy_coded_amd.synth import make_workload
    monkeypatch.setenv("WC_DEBUG", "1")
    wl = make_workload("heavy_tail_14k", scale_rows=96)
    blob = wc.encode_host(wl.tensors(), **enc)
    with wc.Plan(blob) as plan:
        log(f"case: debug plan, valid container {enc}: decode")
        assert np.array_equal(gpu_decode(wc, blob, plan=plan), wl.bits)
        assert wc.plan_debug_status(plan) == 0
        log(f"case: debug plan, valid container {enc}: fused product")
        _, dblob = to_device_aligned(blob)
        ys = _fused(wc, plan, dblob, wl.shapes)
        assert all(np.all(np.isfinite(y)) for y in ys)
        assert wc.plan_debug_status(plan) == 0


@pytest.mark.parametrize("path", ["decode", "fused"])
def test_zero_stream_sets_group_count(wc, monkeypatch, path):
    """A stream of zero bits passes wc_plan's checks (they cover the
    metadata), stays inside its output (the bounds test of corrupted
    streams), and sets WC_DEBUG_GROUP_COUNT; reset clears the word."""
    from lossless_entropy_coded_amd.synth import make_workload
    monkeypatch.setenv("WC_DEBUG", "1")
    wl = make_workload("heavy_tail_14k", scale_rows=96)
    blob = wc.encode_host(wl.tensors(), layout="chunks")
    bad, over = _zero_stream(blob)
    assert over, "no group whose bits exceed L * n: the zero stream proves nothing here"
    with wc.Plan(bad) as plan:
        log(f"case: debug plan, zero stream, {path} ({len(over)} groups over L * n)")
        if path == "decode":
            gpu_decode(wc, bad, plan=plan)      # asserts the guard bands
        else:
            _, dblob = to_device_aligned(bad)
            _fused(wc, plan, dblob, wl.shapes)
        assert wc.plan_debug_status(plan, reset=True) & wc.WC_DEBUG_GROUP_COUNT
        assert wc.plan_debug_status(plan) == 0


def _lane_symbols(m: int) -> np.ndarray:
    """Symbols of each of the 64 lanes of a segment of m elements: lane j takes
    the 8-element lane blocks j, j + 64, ... (the segment's last block may be
    shorter)."""
    nb8 = -(-m // 8)
    nsym = np.array([8 * ((nb8 - 1 - j) // 64 + 1) if j < nb8 else 0 for j in range(64)], dtype=np.int64)
    if nb8:
        nsym[(nb8 - 1) % 64] -= 8 * nb8 - m
    return nsym


def _zero_lanes_stream(blob):
    """A lanes container with every stream byte zero, and the number of lanes
    that provably cannot end their strings where the next ones begin.  Huffman:
    over zero bits every code is the first canonical one (all zeros, the
    shortest length L), and a lane's last table lookup adds at most three
    symbols past its own, so a lane of nsym symbols whose string is longer
    than L (nsym + 3) bits stops short of its end.  rANS: the final state
    read is 0, and from state 0 every step stays at 0 (the first present
    symbol owns slot 0 with cumulative frequency 0, and renormalising shifts
    in zero words), never the initial state 2^16 a lane must end in."""
    from container_view import sections
    s = sections(blob)
    b = blob.copy()
    b[s["off_stream"]:s["off_stream"] + s["stream_bytes"]] = 0
    g = s["groups"].astype(np.int64)
    off = s["lane_off"].astype(np.int64)
    L = None if s["coder"] == 1 else int(s["code_len"][s["code_len"] > 0].min())
    caught = 0
    for k in range(int(s["n_groups"])):
        m, seg_bits = g[k + 1, 0] - g[k, 0], g[k + 1, 1] - g[k, 1]
        lens = np.append(off[k, 1:], seg_bits) - off[k]
        nsym = _lane_symbols(int(m))
        if L is None:
            caught += int(np.sum(nsym > 0))
        else:
            caught += int(np.sum((nsym > 0) & (lens > L * (nsym + 3))))
    return b, caught


@pytest.mark.parametrize("coder", ["huffman", "rans"])
@pytest.mark.parametrize("A,M,B,n", [(8, 4096, 15872, None), (64, 1024, 4096, None), (120, 3960, 15872, None),
                                     (8, 512, 500, None), (8, 4096, 15872, 1), (8, 4096, 15872, 9),
                                     (8, 4096, 15872, 521), (128, 4096, 15872, 70_001)])
def test_lanes_valid_shapes_leave_word_clear(wc, monkeypatch, coder, A, M, B, n):
    """The lane-end check of the lanes layout's plain decode (and, for whole
    matrices, of its fused product) on valid containers of every segment
    shape (empty lanes, a short last block, the last lane's end at the
    segment's end, bit caps down to 500): bit-exact, and the status word
    stays 0."""
    from lossless_entropy_coded_amd.synth import make_workload
    monkeypatch.setenv("WC_DEBUG", "1")
    wl = make_workload("heavy_tail_14k", scale_rows=64)
    data = wl.bits if n is None else wl.bits[:n]
    tensors = wl.tensors() if n is None else [data]
    if coder == "rans":
        B = max(B, 2048 + (97 * A + 7) // 8)       # the rANS writer's least segment bit cap
    blob = wc.encode_host(tensors, coder=coder, group_align=A, group_max_elems=M, seg_max_bits=B)
    with wc.Plan(blob) as plan:
        log(f"case: debug plan, lanes {coder} A={A} M={M} B={B} n={data.size}")
        assert np.array_equal(gpu_decode(wc, blob, plan=plan), data)
        assert wc.plan_debug_status(plan) == 0
        if n is None:
            log(f"case: debug plan, lanes {coder} A={A} M={M} B={B}: fused product")
            _, dblob = to_device_aligned(blob)
            ys = _fused(wc, plan, dblob, wl.shapes)
            assert all(np.all(np.isfinite(y)) for y in ys)
            assert wc.plan_debug_status(plan) == 0


@pytest.mark.parametrize("path", ["decode", "fused"])
@pytest.mark.parametrize("coder", ["huffman", "rans"])
def test_lanes_zero_stream_sets_lane_bits(wc, monkeypatch, coder, path):
    """A lanes container whose stream is all zero bits passes wc_plan (its
    checks cover the metadata), stays inside its output, and sets
    WC_DEBUG_LANE_BITS (and nothing else) in the plain decode and in the
    fused product; reset clears the word."""
    from lossless_entropy_coded_amd.synth import make_workload
    monkeypatch.setenv("WC_DEBUG", "1")
    wl = make_workload("heavy_tail_14k", scale_rows=96)
    blob = wc.encode_host(wl.tensors(), coder=coder)
    bad, caught = _zero_lanes_stream(blob)
    assert caught, "no lane provably misses its end: the zero stream proves nothing here"
    with wc.Plan(bad) as plan:
        log(f"case: debug plan, lanes {coder} zero stream, {path} ({caught} lanes must miss their ends)")
        if path == "decode":
            gpu_decode(wc, bad, plan=plan)      # asserts the guard bands
        else:
            _, dblob = to_device_aligned(bad)
            _fused(wc, plan, dblob, wl.shapes)
        assert wc.plan_debug_status(plan, reset=True) == wc.WC_DEBUG_LANE_BITS
        assert wc.plan_debug_status(plan) == 0
