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
