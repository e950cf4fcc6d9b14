"""GPU tests of the fused decode -> matrix-vector product (wc_decode_gemv_async).

The fused path never writes the decoded weights: each wave decodes one group
and multiplies it by x on chip.  Expected values come from the oracle: its
decoder gives W (and must give back the generated weights), its float64 GEMV
gives y.  The GPU sums in fp32 in a fixed order: a lane adds at most 64
products in sequence (8 merge steps of 8 elements), six butterfly levels add
the 64 lane sums, and a row adds the partials of the groups covering it (at
most cols/A + 2 of them, A = the container's block size), so
|y - y64| <= (64 + 6 + cols/A + 2) * 2^-24 * sum |w x|, to first order, plus
the underflow of products of subnormal weights (at most 2^-150 each).
"""
import zlib

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


def _dev_u16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _bound(W, x, align):
    wf = (W.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    cols = W.shape[1]
    terms = 64 + 6 + -(-cols // align) + 2
    return 1.01 * terms * 2.0 ** -24 * (np.abs(wf) @ np.abs(xf)) + cols * 2.0 ** -149


class Fused:
    """A container on the device plus guarded y / work buffers for one tensor."""

    GUARD = 64

    def __init__(self, wc, blob, plan):
        self.wc, self.plan = wc, plan
        self._own, self.dblob = to_device_aligned(blob)

    def run(self, tensor, cols, x):
        import torch
        rows = self.plan.tensor_numels[tensor] // cols
        _, ng = self.plan.tensor_groups(tensor)
        y = torch.full((rows + self.GUARD,), float("nan"), dtype=torch.float32, device="cuda")
        work = torch.full((2 * ng + self.GUARD,), float("nan"), dtype=torch.float32, device="cuda")
        self.wc.decode_gemv_async(self.plan, self.dblob, tensor, cols, _dev_u16(x), y, work)
        torch.cuda.synchronize()
        yh, wh = y.cpu().numpy(), work.cpu().numpy()
        assert np.all(np.isnan(yh[rows:])), "fused GEMV wrote past y[rows]"
        assert np.all(np.isnan(wh[2 * ng:])), "fused GEMV wrote past its work buffer"
        return yh[:rows]


def _check_tensor(oracle_lib, got, W, x, align):
    ref = oracle_lib.gemv_bf16(W, x)
    err = np.abs(got.astype(np.float64) - ref)
    bound = _bound(W, x, align)
    bad = np.nonzero(~(err <= bound))[0]
    assert bad.size == 0, f"rows {bad[:8]} off by {err[bad[:8]]} > {bound[bad[:8]]}"


# (block size A, group cap M, tensors as (rows, cols) or (n,) vectors); every
# tensor offset is a multiple of 8 and most are not multiples of A, so groups
# straddle tensors and rows.
CASES = [
    ("one_row", 128, 4096, [(1, 4096)]),
    ("ragged_rows", 64, 512, [(40,), (3, 512), (17, 520), (5, 1032)]),
    ("cols_equal_cap", 128, 1024, [(8,), (33, 1024), (64,), (9, 3096)]),
    ("small_blocks", 8, 256, [(24,), (31, 256), (12, 264), (1, 2048)]),
    ("odd_block", 120, 960, [(16,), (21, 960), (7, 1960)]),
]


@pytest.mark.parametrize("name,align,cap,shapes", CASES, ids=[c[0] for c in CASES])
def test_fused_against_oracle(wc, oracle_lib, name, align, cap, shapes):
    from lossless_entropy_coded_amd.synth import f32_to_bf16_rne, gemv_input
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    tensors = []
    for s in shapes:
        n = int(np.prod(s))
        tensors.append(f32_to_bf16_rne(rng.standard_normal(n, dtype=np.float32) * np.float32(0.02)))
    blob = wc.encode_host(tensors, group_align=align, group_max_elems=cap)
    W_all = oracle_lib.decode(blob)
    assert np.array_equal(W_all, np.concatenate(tensors))
    with wc.Plan(blob) as plan:
        f = Fused(wc, blob, plan)
        for k, s in enumerate(shapes):
            if len(s) != 2:
                continue
            rows, cols = s
            off = plan.tensor_offsets[k]
            x = gemv_input(cols)
            log(f"case: fused {name} tensor {k} {rows}x{cols} A={align} M={cap}")
            got = f.run(k, cols, x)
            W = W_all[off:off + rows * cols].reshape(rows, cols)
            _check_tensor(oracle_lib, got, W, x, align)
            again = f.run(k, cols, x)
            assert np.array_equal(got.view(np.uint32), again.view(np.uint32)), "fused GEMV is not deterministic"


@pytest.mark.parametrize("name,rows", [("heavy_tail_14k", 96), ("block_8b", 40), ("block_70b", 24)])
def test_fused_on_workload_shapes(wc, oracle_lib, name, rows):
    """The block workloads, truncated to a few rows per matrix: every matrix
    of the block, read through the fused path, against the oracle."""
    from lossless_entropy_coded_amd.synth import gemv_input, make_workload
    wl = make_workload(name, scale_rows=rows)
    blob = wc.encode_host(wl.tensors())
    with wc.Plan(blob) as plan:
        f = Fused(wc, blob, plan)
        for k, shape in enumerate(wl.shapes):
            if len(shape) != 2:
                continue
            r, c = shape
            off = plan.tensor_offsets[k]
            x = gemv_input(c)
            log(f"case: fused {name} rows={rows} tensor {wl.names[k]} {r}x{c}")
            got = f.run(k, c, x)
            _check_tensor(oracle_lib, got, wl.bits[off:off + r * c].reshape(r, c), x, wc.GROUP_ALIGN)


def test_fused_full_block_8b_sampled(wc, oracle_lib):
    """The full 8B-shape block (the size the benchmark decodes): every matrix
    through the fused path; 48 sampled rows per matrix (first, last and random)
    against the oracle's GEMV of the generated weights."""
    from lossless_entropy_coded_amd.synth import gemv_input, make_workload
    wl = make_workload("block_8b")
    blob = wc.encode_host(wl.tensors())
    rng = np.random.default_rng(8)
    with wc.Plan(blob) as plan:
        f = Fused(wc, blob, plan)
        for k, shape in enumerate(wl.shapes):
            if len(shape) != 2:
                continue
            r, c = shape
            off = plan.tensor_offsets[k]
            x = gemv_input(c)
            log(f"case: fused block_8b full tensor {wl.names[k]} {r}x{c}")
            got = f.run(k, c, x)
            assert np.all(np.isfinite(got))
            sample = np.unique(np.concatenate([[0, r - 1], rng.integers(0, r, 46)]))
            W = wl.bits[off:off + r * c].reshape(r, c)[sample]
            _check_tensor(oracle_lib, got[sample], W, x, wc.GROUP_ALIGN)


def test_fused_argument_checks(wc):
    import torch
    from lossless_entropy_coded_amd.synth import f32_to_bf16_rne
    rng = np.random.default_rng(5)
    # offsets: tensor 1 at 4 (not a multiple of 8), tensor 3 at 2056
    t = [f32_to_bf16_rne(rng.standard_normal(n, dtype=np.float32)) for n in (4, 4 * 512, 4, 4 * 512)]
    blob = wc.encode_host(t + [np.zeros(0, np.uint16)], group_align=64, group_max_elems=512)
    with wc.Plan(blob) as plan:
        _, dblob = to_device_aligned(blob)
        x = torch.zeros(1032, dtype=torch.int16, device="cuda")
        y = torch.zeros(64, dtype=torch.float32, device="cuda")
        work = torch.zeros(2 * plan.stats()["n_groups"], dtype=torch.float32, device="cuda")

        def status(tensor, cols, xp=x, yp=y):
            try:
                wc.decode_gemv_async(plan, dblob, tensor, cols, xp, yp, work)
                torch.cuda.synchronize()
                return wc.WC_OK
            except wc.WCError as e:
                return e.status

        assert plan.tensor_offsets[1] == 4 and plan.tensor_offsets[3] == 2056
        assert status(3, 512) == wc.WC_OK
        assert status(5, 512) == wc.WC_ERR_INVALID_ARG      # no such tensor
        assert status(1, 512) == wc.WC_ERR_INVALID_ARG      # element offset 4: not a multiple of 8
        assert status(3, 500) == wc.WC_ERR_INVALID_ARG      # not a multiple of 8
        assert status(3, 256) == wc.WC_ERR_INVALID_ARG      # shorter than the largest group
        assert status(3, 768) == wc.WC_ERR_INVALID_ARG      # does not divide numel
        assert status(3, 0) == wc.WC_ERR_INVALID_ARG
        assert status(3, 512, xp=x.data_ptr() + 2) == wc.WC_ERR_INVALID_ARG
        assert status(4, 512) == wc.WC_OK                    # empty tensor: no-op
