"""GPU tests of the fused decode -> matrix-vector products (wc_decode_gemv_async).

The fused path never writes the decoded weights: each wave decodes one group
and multiplies it by x on chip.  Expected values come from the oracle: its
decoder gives W (and must give back the generated weights), its float64 GEMV
gives y.  The GPU's order is fixed: each 8-element block is summed by four
bf16 dot2 steps (each within 3 * 2^-24 of the sum of its addends'
magnitudes, so at most 12 * 2^-24 * sum |w x| per block), a lane adds its at
most 8 block sums, six butterfly levels add the 64 lanes, and a row adds the
partials of the groups covering it (at most cols/A + 2, A = the container's
block size), so |y - y64| <= (12 + 8 + 6 + cols/A + 2) * 2^-24 * sum |w x| to
first order, plus the rounding of products below fp32's subnormal range.
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
    terms = 12 + 8 + 6 + -(-cols // align) + 2
    return 1.05 * terms * 2.0 ** -24 * (np.abs(wf) @ np.abs(xf)) + cols * 2.0 ** -148


class Fused:
    """A container on the device; runs the fused product over consecutive
    tensors with guarded y and work buffers."""

    GUARD = 64

    def __init__(self, wc, blob, plan):
        self.wc, self.plan = wc, plan
        self._own, self.dblob = to_device_aligned(blob)

    def run(self, ops):
        """ops: [(tensor, cols, x host bf16)] -> list of host y arrays."""
        import torch
        dev = []
        for t, c, x in ops:
            rows = self.plan.tensor_numels[t] // c
            y = torch.full((rows + self.GUARD,), float("nan"), dtype=torch.float32, device="cuda")
            dev.append((t, c, _dev_u16(x), y, rows))
        cops = [(t, c, xd, y) for t, c, xd, y, _ in dev]
        need = self.wc.decode_gemv_work_bytes(self.plan, cops)
        work = torch.full((need // 4 + 256 + self.GUARD,), float("nan"), dtype=torch.float32, device="cuda")
        skew = (-work.data_ptr()) % 256 // 4
        wview = work[skew:]
        self.wc.decode_gemv_async(self.plan, self.dblob, cops, wview, need)
        torch.cuda.synchronize()
        tail = wview[need // 4:].cpu().numpy()
        assert np.all(np.isnan(tail)), "fused GEMV wrote past its work buffer"
        out = []
        for _, _, _, y, rows in dev:
            yh = y.cpu().numpy()
            assert np.all(np.isnan(yh[rows:])), "fused GEMV wrote past y[rows]"
            out.append(yh[:rows])
        return out


def _check_tensor(oracle_lib, got, W, x, align):
    ref = oracle_lib.gemv_bf16(W, x)
    err = np.abs(got.astype(np.float64) - ref)
    bound = _bound(W, x, align)
    bad = np.nonzero(~(err <= bound))[0]
    assert bad.size == 0, f"rows {bad[:8]} off by {err[bad[:8]]} > {bound[bad[:8]]}"


# the container variants the fused product runs on: Huffman in interleaved
# lanes, Huffman in chunks (byte or packed gaps), rANS in interleaved lanes
# (whose segments are also runs of whole blocks, so the same bound holds)
ENCODINGS = {"lanes": {"layout": "lanes"}, "chunks": {"layout": "chunks"},
             "rans": {"layout": "lanes", "coder": "rans"}, "chunks5": {"layout": "chunks", "gap_bits": 5},
             # groups of 64 chunks, and of 1000 chunks (decoded in passes of 128)
             "chunks_g64": {"layout": "chunks", "chunks_per_group": 64},
             "chunks5_g1000": {"layout": "chunks", "gap_bits": 5, "chunks_per_group": 1000}}


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


@pytest.mark.parametrize("layout", ["lanes", "chunks", "rans", "chunks5", "chunks_g64", "chunks5_g1000"])
@pytest.mark.parametrize("name,align,cap,shapes", CASES, ids=[c[0] for c in CASES])
def test_fused_against_oracle(wc, oracle_lib, name, align, cap, shapes, layout):
    """Each matrix alone, then every run of consecutive matrices in one call:
    the values agree with the oracle, the one-call results equal the
    per-matrix ones, and a repeated call gives the same bits."""
    from lossless_entropy_coded_amd.synth import f32_to_bf16_rne, gemv_input
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    tensors = []
    for s in shapes:
        n = int(np.prod(s))
        tensors.append(f32_to_bf16_rne(rng.standard_normal(n, dtype=np.float32) * np.float32(0.02)))
    blob = wc.encode_host(tensors, group_align=align, group_max_elems=cap, **ENCODINGS[layout])
    W_all = oracle_lib.decode(blob)
    assert np.array_equal(W_all, np.concatenate(tensors))
    with wc.Plan(blob) as plan:
        f = Fused(wc, blob, plan)
        mats = [k for k, s in enumerate(shapes) if len(s) == 2]
        alone = {}
        for k in mats:
            rows, cols = shapes[k]
            off = plan.tensor_offsets[k]
            x = gemv_input(cols)
            log(f"case: fused {layout} {name} tensor {k} {rows}x{cols} A={align} M={cap}")
            got = f.run([(k, cols, x)])[0]
            W = W_all[off:off + rows * cols].reshape(rows, cols)
            _check_tensor(oracle_lib, got, W, x, align)
            again = f.run([(k, cols, x)])[0]
            assert np.array_equal(got.view(np.uint32), again.view(np.uint32)), "fused GEMV is not deterministic"
            alone[k] = got
        # consecutive runs of matrices (vectors between matrices break a run)
        runs, cur = [], []
        for k in range(len(shapes)):
            if len(shapes[k]) == 2:
                cur.append(k)
            else:
                runs.append(cur)
                cur = []
        runs.append(cur)
        for run in runs:
            if len(run) < 2:
                continue
            log(f"case: fused {name} tensors {run} in one call")
            ys = f.run([(k, shapes[k][1], gemv_input(shapes[k][1])) for k in run])
            for k, y in zip(run, ys):
                assert np.array_equal(y, alone[k]), f"tensor {k}: one-call result differs from the per-matrix call"


@pytest.mark.parametrize("layout", ["lanes", "chunks", "rans", "chunks5"])
@pytest.mark.parametrize("name,rows", [("heavy_tail_14k", 96), ("block_8b", 40), ("block_70b", 24)])
def test_fused_on_workload_shapes(wc, oracle_lib, name, rows, layout):
    """The block workloads, truncated to a few rows per matrix: all matrices
    of the block in one fused call, against the oracle."""
    from lossless_entropy_coded_amd.synth import gemv_input, make_workload
    wl = make_workload(name, scale_rows=rows)
    blob = wc.encode_host(wl.tensors(), **ENCODINGS[layout])
    with wc.Plan(blob) as plan:
        f = Fused(wc, blob, plan)
        mats = [k for k, s in enumerate(wl.shapes) if len(s) == 2]
        assert mats == list(range(len(mats)))
        log(f"case: fused {layout} {name} rows={rows} tensors {mats} in one call")
        ys = f.run([(k, wl.shapes[k][1], gemv_input(wl.shapes[k][1])) for k in mats])
        for k, got in zip(mats, ys):
            r, c = wl.shapes[k]
            off = plan.tensor_offsets[k]
            _check_tensor(oracle_lib, got, wl.bits[off:off + r * c].reshape(r, c), gemv_input(c), wc.GROUP_ALIGN)


@pytest.mark.parametrize("layout", ["lanes", "chunks", "rans", "chunks5"])
def test_fused_full_block_8b_sampled(wc, oracle_lib, layout):
    """The full 8B-shape block (the size the benchmark decodes): its 7
    matrices in one fused call; 48 sampled rows per matrix (first, last and
    random) against the oracle's GEMV of the generated weights."""
    from lossless_entropy_coded_amd.synth import gemv_input, make_workload
    wl = make_workload("block_8b")
    blob = wc.encode_host(wl.tensors(), **ENCODINGS[layout])
    rng = np.random.default_rng(8)
    with wc.Plan(blob) as plan:
        f = Fused(wc, blob, plan)
        mats = [k for k, s in enumerate(wl.shapes) if len(s) == 2]
        log(f"case: fused {layout} block_8b full, tensors {mats} in one call")
        ys = f.run([(k, wl.shapes[k][1], gemv_input(wl.shapes[k][1])) for k in mats])
        for k, got in zip(mats, ys):
            r, c = wl.shapes[k]
            off = plan.tensor_offsets[k]
            assert np.all(np.isfinite(got))
            sample = np.unique(np.concatenate([[0, r - 1], rng.integers(0, r, 46)]))
            W = wl.bits[off:off + r * c].reshape(r, c)[sample]
            _check_tensor(oracle_lib, got[sample], W, gemv_input(c), wc.GROUP_ALIGN)


def test_fused_argument_checks(wc):
    import torch
    from lossless_entropy_coded_amd.synth import f32_to_bf16_rne
    rng = np.random.default_rng(5)
    # offsets: tensor 1 at 4 (not a multiple of 8), tensor 3 at 2056, tensor 4 empty, tensor 5 at 4104
    t = [f32_to_bf16_rne(rng.standard_normal(n, dtype=np.float32)) for n in (4, 4 * 512, 4, 4 * 512)]
    t += [np.zeros(0, np.uint16), f32_to_bf16_rne(rng.standard_normal(2 * 512, dtype=np.float32))]
    blob = wc.encode_host(t, group_align=64, group_max_elems=512)
    with wc.Plan(blob) as plan:
        _, dblob = to_device_aligned(blob)
        x = torch.zeros(1032, dtype=torch.int16, device="cuda")
        y = torch.zeros(64, dtype=torch.float32, device="cuda")
        work = torch.zeros(1 << 16, dtype=torch.float32, device="cuda")
        assert work.data_ptr() % 256 == 0

        def status(ops, nbytes=None):
            try:
                need = wc.decode_gemv_work_bytes(plan, ops)
                wc.decode_gemv_async(plan, dblob, ops, work, need if nbytes is None else nbytes)
                torch.cuda.synchronize()
                return wc.WC_OK
            except wc.WCError as e:
                return e.status

        assert plan.tensor_offsets[1] == 4 and plan.tensor_offsets[3] == 2056 and plan.tensor_offsets[5] == 4104
        assert status([(3, 512, x, y)]) == wc.WC_OK
        assert status([(3, 512, x, y), (4, 512, None, None), (5, 512, x, y)]) == wc.WC_OK   # empty one skipped
        assert status([(4, 512, None, None)]) == wc.WC_OK                    # only empty: no-op
        assert status([]) == wc.WC_ERR_INVALID_ARG
        assert status([(6, 512, x, y)]) == wc.WC_ERR_INVALID_ARG            # no such tensor
        assert status([(3, 512, x, y), (5, 512, x, y)]) == wc.WC_ERR_INVALID_ARG   # not consecutive
        assert status([(1, 512, x, y)]) == wc.WC_ERR_INVALID_ARG            # element offset 4
        assert status([(3, 500, x, y)]) == wc.WC_ERR_INVALID_ARG            # not a multiple of 8
        assert status([(3, 256, x, y)]) == wc.WC_ERR_INVALID_ARG            # shorter than the largest group
        assert status([(3, 768, x, y)]) == wc.WC_ERR_INVALID_ARG            # does not divide numel
        assert status([(3, 0, x, y)]) == wc.WC_ERR_INVALID_ARG
        assert status([(3, 512, x.data_ptr() + 2, y)]) == wc.WC_ERR_INVALID_ARG   # x misaligned
        assert status([(3, 512, x, y)], nbytes=8) == wc.WC_ERR_INVALID_ARG   # work too small
        assert status([(3, 512, x, y)] * 17) == wc.WC_ERR_INVALID_ARG       # more than 16 operands


@pytest.fixture(scope="module")
def block_70b():
    from lossless_entropy_coded_amd.synth import make_workload
    log("case: generating the full 70B-shape block (855,638,016 bf16)")
    return make_workload("block_70b")


@pytest.mark.parametrize("layout", ["lanes", "chunks"])
def test_block_70b_full_size_arms(wc, oracle_lib, block_70b, layout):
    """The full 70B-shape block at the size the benchmark times: the whole
    block decoded in one launch equals the generated weights; the GEMV on the
    decoded buffer (arm A) equals the GEMV on the uncompressed weights (arm B)
    bit for bit for all 7 matrices (28672 x 8192 gate/up, 8192 x 28672 down);
    the fused decode -> GEMV of the 7 matrices in one call (arm C) agrees with
    the oracle's float64 GEMV within the derived bound on 48 sampled rows of
    each matrix (first, last and random), and wrote nothing past y or its
    work buffer."""
    import torch
    from gpu_util import GuardedOutput
    from lossless_entropy_coded_amd.synth import gemv_input
    wl = block_70b
    blob = wc.encode_host(wl.tensors(), layout=layout)
    mats = [(k, s[0], s[1]) for k, s in enumerate(wl.shapes) if len(s) == 2]
    assert [(r, c) for _, r, c in mats] == [(8192, 8192), (1024, 8192), (1024, 8192), (8192, 8192),
                                           (28672, 8192), (28672, 8192), (8192, 28672)]
    rng = np.random.default_rng(70)
    with wc.Plan(blob) as plan:
        f = Fused(wc, blob, plan)
        log(f"case: block_70b full, {layout}: whole-block decode")
        out = GuardedOutput(plan.n_elems)
        wc.decode_async(plan, f.dblob, out.out)
        orig = torch.from_numpy(wl.bits.view(np.int16)).cuda()
        torch.cuda.synchronize()
        assert out.guards_intact()
        assert torch.equal(out.out, orig), "decoded block differs from the generated weights"
        xs = {c: gemv_input(c) for _, _, c in mats}
        xd = {c: _dev_u16(x) for c, x in xs.items()}
        for k, r, c in mats:
            log(f"case: block_70b full, {layout}: arms A and B, tensor {k} {r}x{c}")
            off = plan.tensor_offsets[k]
            ya = torch.full((r,), float("nan"), dtype=torch.float32, device="cuda")
            yb = torch.full((r,), float("nan"), dtype=torch.float32, device="cuda")
            wc.gemv_bf16_async(out.out[off:off + r * c], r, c, xd[c], ya)
            wc.gemv_bf16_async(orig[off:off + r * c], r, c, xd[c], yb)
            torch.cuda.synchronize()
            assert bool(torch.isfinite(yb).all())
            assert torch.equal(ya.view(torch.int32), yb.view(torch.int32)), f"tensor {k}: arm A != arm B"
        del out, orig
        torch.cuda.empty_cache()
        log(f"case: block_70b full, {layout}: arm C, 7 matrices in one fused call")
        ys = f.run([(k, c, xs[c]) for k, _, c in mats])
        for (k, r, c), got in zip(mats, ys):
            assert np.all(np.isfinite(got))
            sample = np.unique(np.concatenate([[0, r - 1], rng.integers(0, r, 46)]))
            off = plan.tensor_offsets[k]
            W = wl.bits[off:off + r * c].reshape(r, c)[sample]
            _check_tensor(oracle_lib, got[sample], W, xs[c], wc.GROUP_ALIGN)
