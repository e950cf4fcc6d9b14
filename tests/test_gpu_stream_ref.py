"""The streaming yardstick (wc_stream_reference_async) moves exactly the
bytes it documents: output item j = NOT input item min(floor(j r / 2^32),
ns - 1), r = ceil(ns 2^32 / nd), computed here with Python integers; every
input item is read; nothing outside the output is written."""
import numpy as np
import pytest
import torch

from gpu_util import log

pytestmark = pytest.mark.gpu

GUARD = 4096


@pytest.fixture(scope="module")
def wc():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from lossless_entropy_coded_amd import wc as mod
    return mod


def expected(src_items: np.ndarray, nd: int) -> np.ndarray:
    ns = src_items.shape[0]
    r = -(-(ns << 32) // nd)
    idx = np.minimum((np.arange(nd, dtype=object) * r) >> 32, ns - 1).astype(np.int64)
    assert set(idx.tolist()) == set(range(ns))           # every input item is read
    return ~src_items[idx]


@pytest.mark.parametrize("ns,nd", [(1, 1), (1, 300), (3, 7), (255, 256), (257, 257), (4096, 6000),
                                   (65536, 96000), (262144, 262145), (1000, 1000003)])
def test_stream_reference_items(wc, ns, nd):
    rng = np.random.default_rng(ns * 7 + nd)
    src = rng.integers(0, 2**32, (ns, 4), dtype=np.uint64).astype(np.uint32)
    d_src = torch.from_numpy(src.view(np.int32).reshape(-1)).cuda()
    buf = torch.full((4 * nd + 2 * GUARD,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    dst = buf[GUARD:GUARD + 4 * nd]
    log(f"case: stream reference ns={ns} nd={nd}")
    wc.stream_reference_async(d_src, 16 * ns, dst, 16 * nd)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint32).reshape(nd, 4)
    assert np.array_equal(got, expected(src, nd))
    assert bool((buf[:GUARD] == 0x5A5A5A5A).all()) and bool((buf[GUARD + 4 * nd:] == 0x5A5A5A5A).all())


def test_stream_reference_rejects(wc):
    a = torch.zeros(64, dtype=torch.int32, device="cuda")
    b = torch.zeros(64, dtype=torch.int32, device="cuda")
    for sb, db in ((32, 16), (16, 24), (8, 16), (0, 16)):
        with pytest.raises(wc.WCError) as ei:
            wc.stream_reference_async(a, sb, b, db)
        assert ei.value.status == wc.WC_ERR_INVALID_ARG
    wc.stream_reference_async(a, 0, b, 0)                  # no-op
    torch.cuda.synchronize()
