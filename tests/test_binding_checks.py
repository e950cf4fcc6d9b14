"""The Python binding's checks of tensor arguments, on the CPU.

The C entry points take bare device pointers without sizes, so the binding
must refuse, before any pointer reaches C, a tensor that the kernels would
read or write past: one that is not a CUDA tensor, sits on another device, is
not contiguous, or is smaller than what the call touches.  No GPU is needed:
a stand-in plan fails the test if a call ever gets as far as its native
handle, and stand-in device tensors carry only the attributes the checks
read.
"""
import types

import pytest
import torch


@pytest.fixture(scope="module")
def wc():
    from lossless_entropy_coded_amd import wc as mod
    return mod


class DevTensor:
    """A device tensor as the binding's checks see it (never dereferenced)."""

    def __init__(self, nbytes, cuda=True, index=0, contiguous=True):
        self.is_cuda = cuda
        self.device = types.SimpleNamespace(index=index)
        self._nbytes, self._contiguous = nbytes, contiguous

    def data_ptr(self):
        return 1 << 24

    def is_contiguous(self):
        return self._contiguous

    def numel(self):
        return self._nbytes

    def element_size(self):
        return 1


class ReachedC(Exception):
    pass


class StandInPlan:
    """A bf16 container of 1000 elements in two tensors (empty, 8 x 512)."""
    n_elems = 1000
    n_tensors = 2
    container_bytes = 4096
    device = 0
    tensor_offsets = [0, 0]
    tensor_numels = [0, 8 * 512]

    @property
    def handle(self):
        raise ReachedC()


def _status(fn):
    try:
        fn()
    except ReachedC:
        return "reached C"
    except Exception as e:  # noqa: BLE001
        return getattr(e, "status", repr(e))
    return "returned"


def test_decode_async_checks(wc):
    p = StandInPlan()
    blob, out = DevTensor(4096), DevTensor(2000)
    assert _status(lambda: wc.decode_async(p, blob, out, 0)) == "reached C"
    bad = {
        "blob on the host": (torch.zeros(4096, dtype=torch.uint8), out),
        "blob short": (DevTensor(4095), out),
        "out short": (blob, DevTensor(1999)),
        "out strided": (blob, DevTensor(4000, contiguous=False)),
        "out on another device": (blob, DevTensor(2000, index=1)),
        "out on the host": (blob, torch.zeros(1000, dtype=torch.int16)),
    }
    for what, (b, o) in bad.items():
        assert _status(lambda: wc.decode_async(p, b, o, 0)) == wc.WC_ERR_INVALID_ARG, what


def test_decode_u8_async_checks(wc):
    p = StandInPlan()
    assert _status(lambda: wc.decode_u8_async(p, DevTensor(4096), DevTensor(1000), 0)) == "reached C"
    assert _status(lambda: wc.decode_u8_async(p, DevTensor(4096), DevTensor(999), 0)) == wc.WC_ERR_INVALID_ARG
    assert _status(lambda: wc.decode_u8_async(p, DevTensor(100), DevTensor(1000), 0)) == wc.WC_ERR_INVALID_ARG


def test_gemv_bf16_async_checks(wc):
    ok = (DevTensor(2 * 4 * 64), 4, 64, DevTensor(128), DevTensor(16))
    # the valid call reaches the library, which fails only for want of a device
    assert _status(lambda: wc.gemv_bf16_async(*ok, stream=0)) not in (wc.WC_ERR_INVALID_ARG,)
    for i, small in ((0, DevTensor(511)), (3, DevTensor(127)), (4, DevTensor(15)),
                     (0, DevTensor(512, contiguous=False)), (4, torch.zeros(4))):
        args = list(ok)
        args[i] = small
        assert _status(lambda: wc.gemv_bf16_async(*args, stream=0)) == wc.WC_ERR_INVALID_ARG, (i, small)
    # rows == 0 touches nothing
    assert _status(lambda: wc.gemv_bf16_async(DevTensor(0), 0, 64, DevTensor(0), DevTensor(0), stream=0)) == \
        "returned"


def test_decode_gemv_checks(wc):
    p = StandInPlan()
    blob, x, y, work = DevTensor(4096), DevTensor(1024), DevTensor(32), DevTensor(4096)
    ops = [(0, 512, None, None), (1, 512, x, y)]          # tensor 0 is empty: x, y unused
    assert _status(lambda: wc.decode_gemv_work_bytes(p, ops)) == "reached C"
    assert _status(lambda: wc.decode_gemv_async(p, blob, ops, work, 4096, 0)) == "reached C"
    bad = {
        "x short": [(1, 512, DevTensor(1023), y)],
        "y short": [(1, 512, x, DevTensor(31))],
        "x on the host": [(1, 512, torch.zeros(512, dtype=torch.int16), y)],
        "y strided": [(1, 512, x, DevTensor(64, contiguous=False))],
    }
    for what, o in bad.items():
        assert _status(lambda: wc.decode_gemv_work_bytes(p, o)) == wc.WC_ERR_INVALID_ARG, what
        assert _status(lambda: wc.decode_gemv_async(p, blob, o, work, 4096, 0)) == wc.WC_ERR_INVALID_ARG, what
    assert _status(lambda: wc.decode_gemv_async(p, blob, ops, DevTensor(4095), 4096, 0)) == wc.WC_ERR_INVALID_ARG
    assert _status(lambda: wc.decode_gemv_async(p, DevTensor(10), ops, work, 4096, 0)) == wc.WC_ERR_INVALID_ARG


def test_raw_pointers_pass_through(wc):
    """Integer pointers carry no size: they go to C, which checks alignment."""
    p = StandInPlan()
    assert _status(lambda: wc.decode_async(p, 1 << 24, 1 << 24, 0)) == "reached C"


def test_decode_gemv_noalloc_checks(wc):
    p = StandInPlan()
    blob, x, y = DevTensor(4096), DevTensor(1024), DevTensor(32)
    assert _status(lambda: wc.decode_gemv_noalloc_async(p, blob, [(1, 512, x, y)], 0)) == "reached C"
    assert _status(lambda: wc.decode_gemv_noalloc_async(p, blob, [(1, 512, DevTensor(1000), y)], 0)) == \
        wc.WC_ERR_INVALID_ARG
    assert _status(lambda: wc.decode_gemv_noalloc_async(p, DevTensor(64), [(1, 512, x, y)], 0)) == \
        wc.WC_ERR_INVALID_ARG
