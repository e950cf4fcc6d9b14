"""GPU tests of the batch-1 bf16 GEMV that consumes decoded weights.

The GEMV accumulates in fp32; it is checked against the oracle's float64
product with the rounding bound of its fixed summation order: each lane adds
at most cols/64 + 8 products in sequence, then six butterfly levels add the
lane partials, so |y - y64| <= (cols/64 + 14) * 2^-24 * sum |w x| (first-order
bound of recursive fp32 summation; every bf16 product is exact in fp32).
Decoding a container and multiplying the decoded view must give y bit-identical
to multiplying the original weights (same kernel, same bits).
"""
import numpy as np
import pytest

from gpu_util import GuardedOutput, log, to_device_aligned

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


def _bound(W, x):
    wf = (W.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return (W.shape[1] / 64 + 14) * 2.0 ** -24 * (np.abs(wf) @ np.abs(xf))


def _gemv(wc, W, x):
    import torch
    rows, cols = W.shape
    y = torch.full((rows + 64,), float("nan"), dtype=torch.float32, device="cuda")
    wc.gemv_bf16_async(_dev_u16(W), rows, cols, _dev_u16(x), y)
    torch.cuda.synchronize()
    out = y.cpu().numpy()
    assert np.all(np.isnan(out[rows:])), "GEMV wrote past y[rows]"
    return out[:rows]


@pytest.mark.parametrize("rows,cols", [(1, 8), (3, 8), (5, 24), (16, 512), (17, 520), (64, 1024), (100, 4096),
                                       (7, 8200), (33, 28672)])
def test_gemv_against_oracle(wc, oracle_lib, rows, cols):
    from lossless_entropy_coded_amd.synth import f32_to_bf16_rne, gemv_input
    rng = np.random.default_rng(rows * 100003 + cols)
    W = f32_to_bf16_rne(rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(0.02))
    x = gemv_input(cols)
    log(f"case: gemv {rows}x{cols}")
    got = _gemv(wc, W, x).astype(np.float64)
    ref = oracle_lib.gemv_bf16(W, x)
    assert np.all(np.abs(got - ref) <= _bound(W, x))


def test_gemv_special_values(wc, oracle_lib):
    """Zeros, subnormals, signed values and a row of exactly representable sums."""
    cols = 64
    x = np.full(cols, 0x3F80, np.uint16)                       # ones
    W = np.zeros((4, cols), np.uint16)
    W[1, :] = 0x3F80                                           # row of ones: sum 64 exactly
    W[2, ::2] = 0x4000                                         # 2, -2 alternating: sum 0 exactly
    W[2, 1::2] = 0xC000
    W[3, :] = 0x0001                                           # smallest subnormal
    got = _gemv(wc, W, x)
    assert got[0] == 0.0 and got[1] == 64.0 and got[2] == 0.0
    ref = oracle_lib.gemv_bf16(W, x)
    assert abs(float(got[3]) - ref[3]) <= _bound(W, x)[3]


@pytest.mark.parametrize("name,rows", [("block_70b", 256), ("block_8b", 512)])
def test_decoded_weights_give_identical_gemv(wc, oracle_lib, name, rows):
    """Arm A (decode the block, GEMV each decoded matrix view) equals Arm B
    (GEMV on the uncompressed weights) bit for bit."""
    import torch
    from lossless_entropy_coded_amd.synth import gemv_input, make_workload
    wl = make_workload(name, scale_rows=rows)
    blob = wc.encode_host(wl.tensors())
    with wc.Plan(blob) as plan:
        _, dblob = to_device_aligned(blob)
        out = GuardedOutput(plan.n_elems)
        wc.decode_async(plan, dblob, out.out)
        torch.cuda.synchronize()
        assert out.guards_intact()
        orig = _dev_u16(wl.bits)
        for k, shape in enumerate(wl.shapes):
            if len(shape) != 2:
                continue
            r, c = shape
            off = plan.tensor_offsets[k]
            x = _dev_u16(gemv_input(c))
            ya = torch.empty(r, dtype=torch.float32, device="cuda")
            yb = torch.empty(r, dtype=torch.float32, device="cuda")
            wc.gemv_bf16_async(out.out[off:off + r * c], r, c, x, ya)
            wc.gemv_bf16_async(orig[off:off + r * c], r, c, x, yb)
            torch.cuda.synchronize()
            log(f"case: {name} rows={rows} tensor {wl.names[k]} {r}x{c}")
            assert torch.equal(ya.view(torch.int32), yb.view(torch.int32))
            W = wl.bits[off:off + r * c].reshape(r, c)
            ref = oracle_lib.gemv_bf16(W[:64], gemv_input(c))
            got = ya[:64].cpu().numpy().astype(np.float64)
            assert np.all(np.abs(got - ref) <= _bound(W[:64], gemv_input(c)))


def test_gemv_argument_checks(wc):
    import torch
    W = torch.zeros(64, dtype=torch.int16, device="cuda")
    y = torch.zeros(8, dtype=torch.float32, device="cuda")
    with pytest.raises(wc.WCError) as ei:
        wc.gemv_bf16_async(W, 8, 7, W, y)
    assert ei.value.status == wc.WC_ERR_INVALID_ARG
    with pytest.raises(wc.WCError):
        wc.gemv_bf16_async(W.data_ptr() + 2, 4, 8, W, y)
    wc.gemv_bf16_async(W, 0, 8, W, y)         # rows == 0 is a no-op
