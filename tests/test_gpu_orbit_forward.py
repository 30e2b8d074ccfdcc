"""GPU parity of the OrbitQuant runtime forward against the oracle.

Source: "zerogpu-sdxlTrainer: toolkit/util/orbit_quant.py", OrbitQuantizer.forward:
x_rot = rpbh_forward(x) (checked bit for bit: same fp32 operations in the same
order), then F.linear(x_rot, W', bias) with W' = codebook[code] * row_norm
decoded on the fly. The page leaves the matmul's summation order to the BLAS,
so the linear layer is held to the fp32 bound of a K-term dot product:
  |y - y_ref| <= 2 K u sum_j |x_rot_j W'_j| + u |bias|,  u = 2^-24.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from oracle import orbit_forward as of

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
U = 2.0 ** -24


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import randomized_hadamard_lloyd_amd as m
    return m


def quantized(rows, d, bits, seed, msb=True):
    w = np.random.default_rng(seed).standard_normal((rows, d)).astype(np.float32) * 0.02
    perm, sg = datagen.rpbh_params(d)
    cb = oracle.orbit_codebook(bits, d)
    packed, norms = oracle.orbit_quantize(w, bits, perm, sg, cb, msb_first=msb)
    return perm, sg, cb, packed, norms


def check_linear(tq, x_rot, packed, norms, d, bits, cb, bias=None, msb=True):
    order = tq.TQ_MSB_FIRST if msb else tq.TQ_LSB_FIRST
    y = tq.orbit_linear(torch.from_numpy(x_rot).to(DEV), torch.from_numpy(packed).to(DEV),
                        torch.from_numpy(norms).to(DEV), bits, cb,
                        None if bias is None else torch.from_numpy(bias).to(DEV), bit_order=order)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    ref = of.orbit_linear(x_rot, packed, norms, d, bits, cb, bias, msb_first=msb)
    w = of.orbit_rotated_weight(packed, norms, d, bits, cb, msb).astype(np.float64)
    bound = 2 * d * U * (np.abs(x_rot).astype(np.float64) @ np.abs(w).T)
    if bias is not None:
        bound = bound + U * np.abs(bias)[None, :]
    err = np.abs(got - ref)
    assert np.all(err <= bound + 1e-30), (err.max(), (err / (bound + 1e-30)).max())
    return float((err / (bound + 1e-30)).max())


@pytest.mark.parametrize("d", [96, 256, 1024, 1536, 3072, 4096, 5120, 8192, 12288, 16384])
@pytest.mark.parametrize("rows", [1, 7, 65, 300])
def test_rotate_bit_exact(tq, d, rows):
    x = np.random.default_rng(d + rows).standard_normal((rows, d)).astype(np.float32)
    perm, sg = datagen.rpbh_params(d)
    got = tq.orbit_rotate(torch.from_numpy(x).to(DEV), perm.to(DEV), sg.to(DEV)).cpu().numpy()
    ref = oracle.rpbh_forward(x, perm, sg)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("m", [1, 5, 16, 17, 32, 33, 130, 300])
@pytest.mark.parametrize("d,n,bits,msb", [(96, 100, 2, True), (1024, 129, 3, True),
                                          (3072, 384, 4, False), (3072, 384, 4, True),
                                          (512, 1, 3, False),
                                          (2048, 256, 2, True)])
def test_linear(tq, m, d, n, bits, msb):
    perm, sg, cb, packed, norms = quantized(n, d, bits, d + n + bits, msb)
    x_rot = oracle.rpbh_forward(
        np.random.default_rng(m).standard_normal((m, d)).astype(np.float32), perm, sg)
    bias = np.random.default_rng(n).standard_normal(n).astype(np.float32) if m % 2 else None
    check_linear(tq, x_rot, packed, norms, d, bits, cb, bias, msb)


@pytest.mark.parametrize("bits,rows", [(2, 64), (3, 64), (4, 64), (3, 16), (4, 16)])
def test_forward_config5(tq, bits, rows):
    """The weight workload (12288 x 3072, N(0, 0.02^2)) quantized by the
    oracle; 64 or 16 activation rows through the whole forward."""
    d = 3072
    w = datagen.orbit_weight().numpy()
    perm, sg = datagen.rpbh_params(d)
    cb = oracle.orbit_codebook(bits, d)
    packed, norms = oracle.orbit_quantize(w, bits, perm, sg, cb)
    x = np.random.default_rng(bits + rows).standard_normal((rows, d)).astype(np.float32)
    bias = np.random.default_rng(9).standard_normal(w.shape[0]).astype(np.float32) * 0.1
    y = tq.orbit_forward(torch.from_numpy(x).to(DEV), torch.from_numpy(packed).to(DEV),
                         torch.from_numpy(norms).to(DEV), perm.to(DEV), sg.to(DEV), bits, cb,
                         torch.from_numpy(bias).to(DEV))
    torch.cuda.synchronize()
    x_rot, ref = of.orbit_forward(x, packed, norms, perm.numpy(), sg.numpy(), bits, cb, bias)
    wr = of.orbit_rotated_weight(packed, norms, d, bits, cb).astype(np.float64)
    bound = 2 * d * U * (np.abs(x_rot).astype(np.float64) @ np.abs(wr).T) + U * np.abs(bias)
    err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= bound), (err.max(), (err / bound).max())
    print(f"bits {bits}: max error / bound = {(err / bound).max():.3e}")


@pytest.mark.parametrize("fmt", ["fp32", "bf16"])
def test_forward_large_d(tq, fmt):
    """The whole forward on a down-projection shape: in_features 12288 (the
    transposed config-5 weight, h = 4096), 768 outputs, 3 bits, 40 rows."""
    d, n, bits = 12288, 768, 3
    perm, sg, cb, packed, norms = quantized(n, d, bits, 99)
    x = np.random.default_rng(4).standard_normal((40, d)).astype(np.float32)
    if fmt == "fp32":
        xr = tq.orbit_rotate(torch.from_numpy(x).to(DEV), perm.to(DEV), sg.to(DEV))
        x_rot = oracle.rpbh_forward(x, perm, sg)
        assert np.array_equal(xr.cpu().numpy().view(np.uint32), x_rot.view(np.uint32))
        check_linear(tq, x_rot, packed, norms, d, bits, cb)
    else:
        x = of.round_to(x, fmt)
        xr = tq.orbit_rotate(lp_tensor(x, fmt).to(DEV), perm.to(DEV), sg.to(DEV))
        x_rot = of.rpbh_forward_lowp(x, perm.numpy(), sg.numpy(), fmt)
        assert np.array_equal(xr.float().cpu().numpy().view(np.uint32), x_rot.view(np.uint32))
        check_linear_lowp(tq, fmt, x_rot, packed, norms, d, bits, cb)


def test_argument_errors(tq):
    L = tq.lib
    cb = tq._host_f32([-1.0, -0.5, 0.5, 1.0])
    import ctypes
    p = ctypes.cast(cb, ctypes.c_void_p)
    assert L.orbit_linear(None, 0, 4, 100, None, None, 8, 2, p, 0, None, None, None) == 2  # d_in % 32
    assert L.orbit_linear(None, 0, 4, 96, None, None, 8, 5, p, 0, None, None, None) == 4
    assert L.orbit_linear(None, 0, 0, 96, None, None, 8, 2, p, 0, None, None, None) == 0
    assert L.orbit_linear(None, 0, 4, 96, None, None, 8, 2, p, 0, None, None, None) == 1
    assert L.orbit_linear(None, 5, 4, 96, None, None, 8, 2, p, 0, None, None, None) == 3
    assert L.orbit_rotate(None, 0, 4, 48, None, None, None, None) == 5
    assert L.orbit_rotate(None, 7, 4, 64, None, None, None, None) == 3
    with pytest.raises(ValueError):
        tq.orbit_linear(torch.zeros(3, 96, device=DEV), torch.zeros(10, dtype=torch.uint8, device=DEV),
                        torch.zeros(8, device=DEV), 2, [-1.0, -0.5, 0.5, 1.0])


# ----------------------------------------------- bf16 / fp16 activations ---
# The page's forward in the activation's dtype: the rotation rounds every
# stage to the format (checked bit for bit against the oracle's form of
# it); W' = round(round(codebook) * round(norm)); the matmul accumulates in
# fp32 on the matrix cores (order the library's) and rounds its output once:
#   |y - y_ref| <= E + ulp_fmt(|y_ref| + E),  E = 2 K u sum|x_rot W'| + u |bias|.

from parity_util import narrow_ulp  # noqa: E402

LP = {"bf16": torch.bfloat16, "f16": torch.float16}


def lp_tensor(a, fmt):
    """fp32 values already in the format -> a tensor of that dtype (exact)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(LP[fmt])


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("d", [96, 256, 1024, 1536, 2048, 3072, 4096, 6144, 14336, 16384])
@pytest.mark.parametrize("rows", [1, 7, 300])
def test_rotate_lowp_bit_exact(tq, fmt, d, rows):
    x = of.round_to(np.random.default_rng(d + rows).standard_normal((rows, d)).astype(np.float32)
                    * 3.0, fmt)
    perm, sg = datagen.rpbh_params(d)
    got = tq.orbit_rotate(lp_tensor(x, fmt).to(DEV), perm.to(DEV), sg.to(DEV))
    assert got.dtype == LP[fmt]
    got = got.float().cpu().numpy()
    ref = of.rpbh_forward_lowp(x, perm.numpy(), sg.numpy(), fmt)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("fmt", ["fp32", "bf16", "f16"])
def test_rotate_rows_with_zeros(tq, fmt):
    """Rows that hold exact zeros (half the entries, as after a ReLU) and a
    row of equal entries: the values match the oracle; an exact zero of the
    result may carry the other sign where the input held zeros (the page's
    sign of such a zero follows the signs of the input zeros through every
    stage), and is +0 where the zero is a cancellation of nonzero inputs."""
    d = 1536
    rng = np.random.default_rng(12)
    x = rng.standard_normal((4, d)).astype(np.float32)
    x[:3] *= rng.random((3, d)) < 0.5
    x[3] = 1.0
    perm, sg = datagen.rpbh_params(d)
    if fmt == "fp32":
        got = tq.orbit_rotate(torch.from_numpy(x).to(DEV), perm.to(DEV), sg.to(DEV)).cpu().numpy()
        ref = oracle.rpbh_forward(x, perm, sg)
    else:
        x = of.round_to(x, fmt)
        got = tq.orbit_rotate(lp_tensor(x, fmt).to(DEV), perm.to(DEV), sg.to(DEV))
        got = got.float().cpu().numpy()
        ref = of.rpbh_forward_lowp(x, perm.numpy(), sg.numpy(), fmt)
    assert np.array_equal(got, ref)  # -0 == +0
    assert np.array_equal(got[3].view(np.uint32), ref[3].view(np.uint32))
    assert (ref[3] == 0).sum() > 0  # cancellations of nonzero entries


def check_linear_lowp(tq, fmt, x_rot, packed, norms, d, bits, cb, bias=None, msb=True):
    order = tq.TQ_MSB_FIRST if msb else tq.TQ_LSB_FIRST
    y = tq.orbit_linear(lp_tensor(x_rot, fmt).to(DEV), torch.from_numpy(packed).to(DEV),
                        torch.from_numpy(norms).to(DEV), bits, cb,
                        None if bias is None else lp_tensor(bias, fmt).to(DEV), bit_order=order)
    torch.cuda.synchronize()
    assert y.dtype == LP[fmt]
    got = y.float().cpu().numpy().astype(np.float64)
    w = of.orbit_rotated_weight_lowp(packed, norms, d, bits, cb, fmt, msb).astype(np.float64)
    ref = x_rot.astype(np.float64) @ w.T
    E = 2 * d * U * (np.abs(x_rot).astype(np.float64) @ np.abs(w).T)
    if bias is not None:
        ref = ref + bias.astype(np.float64)[None, :]
        E = E + U * np.abs(bias)[None, :]
    bound = E + narrow_ulp((np.abs(ref) + E).astype(np.float32), LP[fmt])
    err = np.abs(got - ref)
    assert np.all(err <= bound), (err.max(), (err / bound).max())
    return float((err / bound).max())


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("m", [1, 5, 20, 40, 64, 130, 300])
@pytest.mark.parametrize("d,n,bits,msb", [(96, 100, 2, True), (1024, 129, 3, True),
                                          (3072, 384, 4, False), (3072, 384, 4, True),
                                          (512, 1, 3, False),
                                          (2048, 256, 2, True)])
def test_linear_lowp(tq, fmt, m, d, n, bits, msb):
    perm, sg, cb, packed, norms = quantized(n, d, bits, d + n + bits, msb)
    x = of.round_to(np.random.default_rng(m).standard_normal((m, d)).astype(np.float32), fmt)
    x_rot = of.rpbh_forward_lowp(x, perm.numpy(), sg.numpy(), fmt)
    bias = (of.round_to(np.random.default_rng(n).standard_normal(n).astype(np.float32), fmt)
            if m % 2 else None)
    check_linear_lowp(tq, fmt, x_rot, packed, norms, d, bits, cb, bias, msb)


def test_linear_lowp_many_row_tiles(tq):
    """1024 rows (four 256-row tiles) at the forward workload's width."""
    perm, sg, cb, packed, norms = quantized(384, 3072, 3, 77)
    x = of.round_to(np.random.default_rng(5).standard_normal((1024, 3072)).astype(np.float32),
                    "bf16")
    x_rot = of.rpbh_forward_lowp(x, perm.numpy(), sg.numpy(), "bf16")
    check_linear_lowp(tq, "bf16", x_rot, packed, norms, 3072, 3, cb)


@pytest.mark.parametrize("fmt,m,d,n,bits,msb", [
    ("bf16", 257, 96, 65, 3, True),     # a row tile holding one row, a half step, a lone column
    ("f16", 520, 160, 130, 4, False),   # three row tiles, two and a half steps
    ("bf16", 300, 64, 1, 2, True),      # a single step, a single output column
    ("f16", 65, 3072, 200, 2, False),   # the fewest rows that take 256 x 64 tiles
    ("bf16", 1000, 1024, 64, 3, False),  # LSB-first 3-bit codes
])
def test_linear_lowp_tall_tiles(tq, fmt, m, d, n, bits, msb):
    """More than 64 rows: 256 x 64 tiles of y, with rows and columns past the
    ends, K an odd multiple of 32 and a one-step K."""
    perm, sg, cb, packed, norms = quantized(n, d, bits, d + n + bits + m, msb)
    x = of.round_to(np.random.default_rng(m + d).standard_normal((m, d)).astype(np.float32), fmt)
    x_rot = of.rpbh_forward_lowp(x, perm.numpy(), sg.numpy(), fmt)
    bias = of.round_to(np.random.default_rng(n).standard_normal(n).astype(np.float32), fmt)
    check_linear_lowp(tq, fmt, x_rot, packed, norms, d, bits, cb, bias, msb)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_forward_lowp_config5(tq, fmt):
    """The 12288 x 3072 weight at 3 bits; 64 activation rows of the format
    through the whole forward (rotation bit for bit, then the linear layer)."""
    d, bits = 3072, 3
    w = datagen.orbit_weight().numpy()
    perm, sg = datagen.rpbh_params(d)
    cb = oracle.orbit_codebook(bits, d)
    packed, norms = oracle.orbit_quantize(w, bits, perm, sg, cb)
    x = of.round_to(np.random.default_rng(3).standard_normal((64, d)).astype(np.float32), fmt)
    bias = of.round_to(np.random.default_rng(9).standard_normal(w.shape[0]).astype(np.float32)
                       * 0.1, fmt)
    xr = tq.orbit_rotate(lp_tensor(x, fmt).to(DEV), perm.to(DEV), sg.to(DEV))
    x_rot = of.rpbh_forward_lowp(x, perm.numpy(), sg.numpy(), fmt)
    assert np.array_equal(xr.float().cpu().numpy().view(np.uint32), x_rot.view(np.uint32))
    r = check_linear_lowp(tq, fmt, x_rot, packed, norms, d, bits, cb, bias)
    print(f"{fmt}: max error / bound = {r:.3e}")


def test_lowp_argument_errors(tq):
    x = torch.zeros(3, 96, dtype=torch.bfloat16, device=DEV)
    pk = torch.zeros(8 * 96 * 2 // 8, dtype=torch.uint8, device=DEV)
    nr = torch.ones(8, device=DEV)
    with pytest.raises(ValueError):  # bias of another dtype
        tq.orbit_linear(x, pk, nr, 2, [-1.0, -0.5, 0.5, 1.0], bias=torch.zeros(8, device=DEV))
    with pytest.raises(ValueError):  # out of another dtype
        tq.orbit_linear(x, pk, nr, 2, [-1.0, -0.5, 0.5, 1.0],
                        out=torch.empty(3, 8, device=DEV))


@pytest.mark.parametrize("m", [1, 20, 130])
@pytest.mark.parametrize("d", [32, 64, 96, 160])
def test_linear_lowp_short_k(tq, m, d):
    """K of one to five 32-wide steps: fewer steps than the few-rows kernel
    has waves, and an odd number of 32-column halves for the many-rows one."""
    perm, sg, cb, packed, norms = quantized(48, d, 3, d + m)
    x = of.round_to(np.random.default_rng(m + d).standard_normal((m, d)).astype(np.float32), "bf16")
    x_rot = of.rpbh_forward_lowp(x, perm.numpy(), sg.numpy(), "bf16")
    check_linear_lowp(tq, "bf16", x_rot, packed, norms, d, 3, cb)
