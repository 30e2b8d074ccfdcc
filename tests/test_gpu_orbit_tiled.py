"""GPU tests of the forward's tiled path: orbit_rotate_tiled, orbit_linear_tiled
and orbit_forward above 64 bf16 / fp16 rows.

Source: "zerogpu-sdxlTrainer: toolkit/util/orbit_quant.py", OrbitQuantizer.forward
(rpbh_forward, then F.linear with W'). The tiled layout is the library's
(include/tq.h): rows padded to a multiple of 16 with zeros, 1 KB per 16 rows x
32 columns, lane l's 8 elements at l * 8 holding row l % 16, columns
8 (l / 16) .. + 7.

* The tiled rotation is the oracle's rotation in the format
  (oracle.orbit_forward.rpbh_forward_lowp), re-tiled here on the host, bit for
  bit, pad rows included.
* The tiled linear layer reads a host-tiled copy of the oracle's x_rot and is
  held to the fp32 dot-product bound of the other forward tests; it must also
  equal orbit_linear on the same rows bit for bit (both run the same MFMAs on
  the same operands in the same order: a check that the two library paths
  agree, beside the oracle bound).
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from oracle import orbit_forward as of
from parity_util import narrow_ulp

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
U = 2.0 ** -24
LP = {"bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import randomized_hadamard_lloyd_amd as m
    return m


def lp_tensor(a, fmt):
    """fp32 values already in the format -> a tensor of that dtype (exact)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(LP[fmt])


def tile_host(x):
    """[m, d] -> the flat tiled order: fragment (t, kc) at (t * d/32 + kc) * 512
    elements, lane l = 16 g + r of it at l * 8: row 16 t + r, columns
    32 kc + 8 g .. + 7; rows padded to a multiple of 16 with zeros."""
    m, d = x.shape
    mp = (m + 15) // 16 * 16
    xp = np.zeros((mp, d), dtype=x.dtype)
    xp[:m] = x
    t = xp.reshape(mp // 16, 16, d // 32, 4, 8)   # [t, r, kc, g, e]
    return np.ascontiguousarray(t.transpose(0, 2, 3, 1, 4)).reshape(-1)


def quantized(rows, d, bits, seed, msb=True):
    w = np.random.default_rng(seed).standard_normal((rows, d)).astype(np.float32) * 0.02
    perm, sg = datagen.rpbh_params(d)
    cb = oracle.orbit_codebook(bits, d)
    packed, norms = oracle.orbit_quantize(w, bits, perm, sg, cb, msb_first=msb)
    return perm, sg, cb, packed, norms


def check_bound(got, x_rot, packed, norms, d, bits, cb, fmt, bias=None, msb=True):
    """|y - y_ref| <= E + ulp_fmt(|y_ref| + E), E = 2 K u sum|x_rot W'| + u |bias|."""
    got = got.astype(np.float64)
    w = of.orbit_rotated_weight_lowp(packed, norms, d, bits, cb, fmt, msb).astype(np.float64)
    ref = x_rot.astype(np.float64) @ w.T
    E = 2 * d * U * (np.abs(x_rot).astype(np.float64) @ np.abs(w).T)
    if bias is not None:
        ref = ref + bias.astype(np.float64)[None, :]
        E = E + U * np.abs(bias)[None, :]
    bound = E + narrow_ulp((np.abs(ref) + E).astype(np.float32), LP[fmt])
    err = np.abs(got - ref)
    assert np.all(err <= bound), (err.max(), (err / bound).max())


def test_tile_host_layout():
    """The host re-tiling puts element (r, k) where the layout says."""
    m, d = 37, 96
    x = np.arange(m * d, dtype=np.float32).reshape(m, d) + 1
    flat = tile_host(x)
    assert flat.size == 48 * d
    for r, k in [(0, 0), (5, 7), (15, 8), (16, 31), (36, 95), (20, 40)]:
        t, kc, g = r // 16, k // 32, (k % 32) // 8
        lane = 16 * g + r % 16
        assert flat[(t * (d // 32) + kc) * 512 + lane * 8 + k % 8] == x[r, k]
    assert (flat != 0).sum() == m * d   # the 11 pad rows are zero


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("m,d", [(1, 64), (17, 96), (100, 1024), (65, 2048), (300, 3072),
                                 (33, 4096), (20, 12288)])
def test_rotate_tiled_bit_exact(tq, fmt, m, d):
    x = of.round_to(np.random.default_rng(m + d).standard_normal((m, d)).astype(np.float32)
                    * 2.0, fmt)
    perm, sg = datagen.rpbh_params(d)
    xt = torch.full((tq.orbit_tiled_bytes(m, d) // 2,), float("nan"), dtype=LP[fmt], device=DEV)
    got = tq.orbit_rotate_tiled(lp_tensor(x, fmt).to(DEV), perm.to(DEV), sg.to(DEV), out=xt)
    assert got.data_ptr() == xt.data_ptr() and got.numel() * 2 == tq.orbit_tiled_bytes(m, d)
    ref = tile_host(of.rpbh_forward_lowp(x, perm.numpy(), sg.numpy(), fmt))
    got = got.float().cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))   # pad rows +0 too


@pytest.mark.parametrize("fmt,m,d,n,bits,msb", [
    ("bf16", 1, 64, 40, 3, True),        # one row: a single row tile, a single step
    ("f16", 20, 96, 65, 2, False),       # a half step, a lone output column
    ("bf16", 64, 160, 130, 4, True),     # two and a half steps
    ("f16", 257, 96, 65, 3, True),       # a row tile holding one row
    ("bf16", 520, 1024, 64, 3, False),   # three 256-row tiles, LSB-first 3-bit codes
    ("f16", 300, 2048, 256, 4, False),
    ("bf16", 1024, 3072, 384, 3, True),  # the forward workload's width, four row tiles
    ("bf16", 100, 96, 65, 3, True),      # steps split in two halves, the second a half step
    ("f16", 200, 224, 130, 2, False),    # four steps in two halves, the last a half step
])
def test_linear_tiled(tq, fmt, m, d, n, bits, msb):
    perm, sg, cb, packed, norms = quantized(n, d, bits, d + n + bits + m, msb)
    x = of.round_to(np.random.default_rng(m + d).standard_normal((m, d)).astype(np.float32), fmt)
    x_rot = of.rpbh_forward_lowp(x, perm.numpy(), sg.numpy(), fmt)
    bias = (of.round_to(np.random.default_rng(n).standard_normal(n).astype(np.float32), fmt)
            if m % 2 == 0 else None)
    order = tq.TQ_MSB_FIRST if msb else tq.TQ_LSB_FIRST
    pk, nr = torch.from_numpy(packed).to(DEV), torch.from_numpy(norms).to(DEV)
    bt = None if bias is None else lp_tensor(bias, fmt).to(DEV)
    y_t = tq.orbit_linear_tiled(lp_tensor(tile_host(x_rot), fmt).to(DEV), m, pk, nr, bits, cb,
                                bt, bit_order=order)
    y_r = tq.orbit_linear(lp_tensor(x_rot, fmt).to(DEV), pk, nr, bits, cb, bt, bit_order=order)
    torch.cuda.synchronize()
    assert y_t.shape == (m, n) and y_t.dtype == LP[fmt]
    got = y_t.float().cpu().numpy()
    check_bound(got, x_rot, packed, norms, d, bits, cb, fmt, bias, msb)
    assert np.array_equal(got.view(np.uint32), y_r.float().cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("m", [65, 300])
def test_forward_tiled_path(tq, fmt, m):
    """orbit_forward above 64 rows (the tiled path): the oracle bound, and the
    same bits as rotate + linear on the row-major path."""
    d, n, bits = 3072, 256, 3
    perm, sg, cb, packed, norms = quantized(n, d, bits, 41 + m)
    x = of.round_to(np.random.default_rng(m).standard_normal((2, (m + 1) // 2, d))
                    .astype(np.float32), fmt)
    rows = x.shape[0] * x.shape[1]
    assert rows > 64
    bias = of.round_to(np.random.default_rng(5).standard_normal(n).astype(np.float32), fmt)
    args = (torch.from_numpy(packed).to(DEV), torch.from_numpy(norms).to(DEV))
    xd = lp_tensor(x, fmt).to(DEV)
    y = tq.orbit_forward(xd, *args, perm.to(DEV), sg.to(DEV), bits, cb,
                         lp_tensor(bias, fmt).to(DEV))
    assert y.shape == (*x.shape[:-1], n)
    y2 = tq.orbit_linear(tq.orbit_rotate(xd, perm.to(DEV), sg.to(DEV)), *args, bits, cb,
                         lp_tensor(bias, fmt).to(DEV))
    torch.cuda.synchronize()
    got = y.float().cpu().numpy().reshape(rows, n)
    x_rot = of.rpbh_forward_lowp(x.reshape(rows, d), perm.numpy(), sg.numpy(), fmt)
    check_bound(got, x_rot, packed, norms, d, bits, cb, fmt, bias)
    assert np.array_equal(got.view(np.uint32),
                          y2.float().cpu().numpy().reshape(rows, n).view(np.uint32))


def test_tiled_argument_errors(tq):
    d = 96
    perm, sg = datagen.rpbh_params(d)
    cb = [-1.0, -0.5, 0.5, 1.0]
    with pytest.raises(ValueError):   # fp32 has no tiled form
        tq.orbit_rotate_tiled(torch.zeros(4, d, device=DEV), perm.to(DEV), sg.to(DEV))
    with pytest.raises(ValueError):   # out of the wrong size
        tq.orbit_rotate_tiled(torch.zeros(4, d, dtype=torch.bfloat16, device=DEV), perm.to(DEV),
                              sg.to(DEV), out=torch.empty(4 * d, dtype=torch.bfloat16,
                                                          device=DEV))
    pk = torch.zeros(8 * d * 2 // 8, dtype=torch.uint8, device=DEV)
    nr = torch.ones(8, device=DEV)
    xt = torch.zeros(tq.orbit_tiled_bytes(4, d) // 2, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):   # m that does not match the buffer
        tq.orbit_linear_tiled(xt, 17, pk, nr, 2, cb)
    pk32 = torch.zeros(8 * 32 * 2 // 8, dtype=torch.uint8, device=DEV)
    xt32 = torch.zeros(tq.orbit_tiled_bytes(4, 32) // 2, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):   # d_in = 32: no tall tiles (TQ_ERR_SHAPE)
        tq.orbit_linear_tiled(xt32, 4, pk32, nr, 2, cb)
    assert tq.orbit_tiled_bytes(4, 48) == 0 and tq.orbit_tiled_bytes(17, 64) == 32 * 64 * 2
