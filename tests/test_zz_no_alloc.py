"""GPU tests of wc_decode_gemv_noalloc_async, the fused decode -> GEMV entry
point that allocates nothing (its work buffer is the library's static device
array), through the C ABI.

Its launches are those of wc_decode_gemv_async, whose results are a
deterministic function of the weights and x, so the bar is bit-identity with
wc_decode_gemv_async on a caller's buffer: on two calls in a row, the second
with a smaller input (the array keeps the first call's contents), and a third
repeating the first.  Work beyond the array's size is refused.
"""
import numpy as np
import pytest

from gpu_util import log, to_device_aligned

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wc():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from lossless_entropy_coded_amd import wc as mod
    return mod


GUARD = 64


def _both(wc, plan, dblob, ops):
    """y of every operand (tensor, cols, x host) from the caller-buffer entry
    point and from the no-allocation one, with NaN guards after each y."""
    import torch
    xs = [torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda() for _, _, x in ops]
    rows = [plan.tensor_numels[t] // c for t, c, _ in ops]
    ya = [torch.full((r + GUARD,), float("nan"), dtype=torch.float32, device="cuda") for r in rows]
    yb = [torch.full((r + GUARD,), float("nan"), dtype=torch.float32, device="cuda") for r in rows]
    ops_a = [(t, c, x, y) for (t, c, _), x, y in zip(ops, xs, ya)]
    ops_b = [(t, c, x, y) for (t, c, _), x, y in zip(ops, xs, yb)]
    need = wc.decode_gemv_work_bytes(plan, ops_a)
    assert 0 < need <= wc.NOALLOC_SCRATCH_BYTES
    work = torch.empty(need // 4 + 64, dtype=torch.float32, device="cuda")
    work = work[(-work.data_ptr()) % 256 // 4:]
    wc.decode_gemv_async(plan, dblob, ops_a, work, need)
    wc.decode_gemv_noalloc_async(plan, dblob, ops_b)
    torch.cuda.synchronize()
    out = []
    for a, b, r in zip(ya, yb, rows):
        a, b = a.cpu().numpy(), b.cpu().numpy()
        assert np.all(np.isnan(b[r:])), "the no-allocation call wrote past y"
        assert np.all(np.isfinite(b[:r]))
        out.append((a[:r], b[:r]))
    return out


def test_noalloc_equals_caller_buffer_on_consecutive_calls(wc):
    from lossless_entropy_coded_amd.synth import gemv_input, make_workload
    big = make_workload("block_8b", scale_rows=256)                 # 7 matrices of 256 rows
    small = make_workload("heavy_tail_14k", scale_rows=40)           # one 40 x 4096 matrix
    cases = [("block_8b, 256 rows per matrix, lanes", big, "lanes"),
             ("heavy_tail_14k, 40 rows, chunks (smaller)", small, "chunks"),
             ("block_8b, 256 rows per matrix, lanes (again)", big, "lanes")]
    for desc, wl, layout in cases:
        blob = wc.encode_host(wl.tensors(), layout=layout)
        with wc.Plan(blob) as plan:
            _, dblob = to_device_aligned(blob)
            mats = [k for k, s in enumerate(wl.shapes) if len(s) == 2]
            ops = [(k, wl.shapes[k][1], gemv_input(wl.shapes[k][1])) for k in mats]
            log(f"case: no-allocation fused GEMV, {desc}: {len(ops)} matrices")
            for k, (a, b) in zip(mats, _both(wc, plan, dblob, ops)):
                assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{desc}: tensor {k} differs"


def test_noalloc_refuses_work_beyond_its_array(wc):
    """A chunks container of 8-element groups: 1,048,576 groups need 8 MiB of
    partials plus 4 bytes per row, more than the array holds."""
    import torch
    from lossless_entropy_coded_amd.synth import f32_to_bf16_rne
    rows, cols = 8192, 1024
    w = f32_to_bf16_rne(np.random.default_rng(9).standard_normal(rows * cols, dtype=np.float32) * np.float32(0.02))
    blob = wc.encode_host([w], layout="chunks", group_align=8, group_max_elems=8)
    with wc.Plan(blob) as plan:
        assert plan.stats()["n_groups"] == rows * cols // 8
        _, dblob = to_device_aligned(blob)
        x = torch.zeros(cols, dtype=torch.int16, device="cuda")
        y = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
        ops = [(0, cols, x, y)]
        assert wc.decode_gemv_work_bytes(plan, ops) > wc.NOALLOC_SCRATCH_BYTES
        log("case: no-allocation fused GEMV beyond the static array")
        with pytest.raises(wc.WCError) as e:
            wc.decode_gemv_noalloc_async(plan, dblob, ops)
        assert e.value.status == wc.WC_ERR_SCRATCH
        torch.cuda.synchronize()
        assert bool(torch.isnan(y).all()), "a refused call wrote y"
