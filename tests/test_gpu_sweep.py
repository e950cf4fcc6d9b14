"""GPU decode of the seeded option sweep (tests/test_writer_sweep.py): every
container the product's writer produces is taken by wc_plan and decodes
bit-exactly to its input through the C ABI, with guard bands; the oracle's
containers for options the product's writer refuses are refused by wc_plan
with WC_ERR_UNSUPPORTED."""
import numpy as np
import pytest
import torch

from gpu_util import gpu_decode, log, to_device_aligned
from test_writer_sweep import CASES, build_case

pytestmark = pytest.mark.gpu

CANARY8 = 0xA5
GUARD8 = 512


@pytest.fixture(scope="module")
def wc():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from lossless_entropy_coded_amd import wc as mod
    return mod


def _decode_u8(wc, blob):
    with wc.Plan(blob) as plan:
        _, dblob = to_device_aligned(blob)
        buf = torch.full((plan.n_elems + 2 * GUARD8,), CANARY8, dtype=torch.uint8, device="cuda")
        out = buf[GUARD8:GUARD8 + plan.n_elems]
        wc.decode_u8_async(plan, dblob, out)
        torch.cuda.synchronize()
        assert bool((buf[:GUARD8] == CANARY8).all()) and bool((buf[GUARD8 + plan.n_elems:] == CANARY8).all())
        return out.cpu().numpy()


def test_sweep_decodes_on_gpu(wc, oracle_lib):
    decoded = refused = 0
    for case in CASES:
        a, b, data, kind, desc = build_case(wc, oracle_lib, case)
        if a is None:
            with pytest.raises(wc.WCError) as ei:
                wc.Plan(b).close()
            assert ei.value.status == wc.WC_ERR_UNSUPPORTED, desc
            refused += 1
            continue
        log(f"case: sweep #{case} {desc}")
        got = _decode_u8(wc, a) if kind == "u8" else gpu_decode(wc, a)
        assert np.array_equal(got, data), f"case {case}: {desc}"
        decoded += 1
    log(f"sweep: {decoded} decoded, {refused} oracle-only containers refused as unsupported")
    assert decoded >= len(CASES) // 2
