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


@pytest.mark.parametrize("d", [96, 256, 1024, 1536, 3072, 4096])
@pytest.mark.parametrize("rows", [1, 7, 65, 300])
def test_rotate_bit_exact(tq, d, rows):
    x = np.random.default_rng(d + rows).standard_normal((rows, d)).astype(np.float32)
    perm, sg = datagen.rpbh_params(d)
    got = tq.orbit_rotate(torch.from_numpy(x).to(DEV), perm.to(DEV), sg.to(DEV)).cpu().numpy()
    ref = oracle.rpbh_forward(x, perm, sg)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("m", [1, 5, 32, 33, 130, 300])
@pytest.mark.parametrize("d,n,bits,msb", [(96, 100, 2, True), (1024, 129, 3, True),
                                          (3072, 384, 4, False), (512, 1, 3, False),
                                          (2048, 256, 2, True)])
def test_linear(tq, m, d, n, bits, msb):
    perm, sg, cb, packed, norms = quantized(n, d, bits, d + n + bits, msb)
    x_rot = oracle.rpbh_forward(
        np.random.default_rng(m).standard_normal((m, d)).astype(np.float32), perm, sg)
    bias = np.random.default_rng(n).standard_normal(n).astype(np.float32) if m % 2 else None
    check_linear(tq, x_rot, packed, norms, d, bits, cb, bias, msb)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_forward_config5(tq, bits):
    """The weight workload (12288 x 3072, N(0, 0.02^2)) quantized by the
    oracle; 64 activation rows through the whole forward."""
    d = 3072
    w = datagen.orbit_weight().numpy()
    perm, sg = datagen.rpbh_params(d)
    cb = oracle.orbit_codebook(bits, d)
    packed, norms = oracle.orbit_quantize(w, bits, perm, sg, cb)
    x = np.random.default_rng(bits).standard_normal((64, d)).astype(np.float32)
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


def test_argument_errors(tq):
    L = tq.lib
    cb = tq._host_f32([-1.0, -0.5, 0.5, 1.0])
    import ctypes
    p = ctypes.cast(cb, ctypes.c_void_p)
    assert L.orbit_linear(None, 4, 100, None, None, 8, 2, p, 0, None, None, None) == 2  # d_in % 32
    assert L.orbit_linear(None, 4, 96, None, None, 8, 5, p, 0, None, None, None) == 4
    assert L.orbit_linear(None, 0, 96, None, None, 8, 2, p, 0, None, None, None) == 0
    assert L.orbit_linear(None, 4, 96, None, None, 8, 2, p, 0, None, None, None) == 1
    assert L.orbit_rotate(None, 4, 48, None, None, None, None) == 5
    with pytest.raises(ValueError):
        tq.orbit_linear(torch.zeros(3, 96, device=DEV), torch.zeros(10, dtype=torch.uint8, device=DEV),
                        torch.zeros(8, device=DEV), 2, [-1.0, -0.5, 0.5, 1.0])
