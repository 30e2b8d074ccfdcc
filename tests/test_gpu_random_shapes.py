"""Parity against the oracle over seeded random shapes.

The launchers pick among many kernel instantiations by shape (several short
rows per wave, blocks of 1-16 waves, stage classes h < 1024 / = 1024 / > 1024,
symmetric and general codebooks, the TQ3 loops by vector count, the linear
layer's few-rows, tall, square and tiled kernels). The fixed-shape tests reach
each of them; these draw many more shapes from a seeded generator, so that a
shape-dependent mistake (an index, a bound, a lane mapping) has more places
to show. Every case is compared with the oracle under the same contract as
the fixed-shape tests.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from oracle import orbit_forward as of
from parity_util import compare_reconstruction, compare_tq3_records, split_records
from test_gpu_orbit import check as orbit_check
from test_gpu_orbit_forward import check_linear_lowp, lp_tensor

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import randomized_hadamard_lloyd_amd as m
    return m


def orbit_shapes(n, seed):
    """(d, rows, bits, msb): d a multiple of 32 up to 16384 (every h from 32),
    rows so that the oracle stays quick."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        kind = rng.integers(0, 4)
        if kind == 0:
            d = 32 * int(rng.integers(1, 17))            # up to 512: several rows per wave
        elif kind == 1:
            d = 32 * int(rng.integers(17, 129))          # up to 4096
        elif kind == 2:
            d = 1024 * int(rng.integers(4, 17))          # wide rows, h from 1024 up
        else:
            d = 32 * int(rng.integers(129, 513))         # wide rows, any h
        rows = int(rng.integers(1, max(2, min(300, (1 << 20) // d))))
        out.append((d, rows, int(rng.integers(2, 5)), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("d,rows,bits,msb", orbit_shapes(40, 2024))
def test_orbit_codec_random_shapes(tq, d, rows, bits, msb):
    w = datagen.orbit_weight(rows=rows, d=d, seed=d * 7 + rows)
    orbit_check(tq, w, d, bits, msb)


@pytest.mark.parametrize("d,rows,bits,msb", orbit_shapes(16, 77))
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_rotation_random_shapes(tq, d, rows, bits, msb, fmt):
    """bf16 / fp16 rotation, row-major and tiled, bit for bit."""
    x = of.round_to(np.random.default_rng(d + rows).standard_normal((rows, d))
                    .astype(np.float32), fmt)
    perm, sg = datagen.rpbh_params(d)
    ref = of.rpbh_forward_lowp(x, perm.numpy(), sg.numpy(), fmt)
    got = tq.orbit_rotate(lp_tensor(x, fmt).to(DEV), perm.to(DEV), sg.to(DEV))
    assert np.array_equal(got.float().cpu().numpy().view(np.uint32), ref.view(np.uint32))
    got_t = tq.orbit_rotate_tiled(lp_tensor(x, fmt).to(DEV), perm.to(DEV), sg.to(DEV))
    mp = (rows + 15) // 16 * 16
    pad = np.zeros((mp, d), np.float32)
    pad[:rows] = ref
    tiled = np.ascontiguousarray(pad.reshape(mp // 16, 16, d // 32, 4, 8)
                                 .transpose(0, 2, 3, 1, 4)).reshape(-1)
    assert np.array_equal(got_t.float().cpu().numpy().view(np.uint32), tiled.view(np.uint32))


def linear_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = 32 * int(rng.integers(1, 65))
        m = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, 400))]))
        out.append((m, d, int(rng.integers(1, 300)), int(rng.integers(2, 5)),
                    bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("m,d,n,bits,msb", linear_shapes(24, 11))
def test_linear_lowp_random_shapes(tq, m, d, n, bits, msb):
    """bf16 linear layer (few-rows, tall and square kernels) and, where it
    applies, the tiled path through orbit_forward."""
    w = np.random.default_rng(d + n).standard_normal((n, d)).astype(np.float32) * 0.02
    perm, sg = datagen.rpbh_params(d)
    cb = oracle.orbit_codebook(bits, d)
    packed, norms = oracle.orbit_quantize(w, bits, perm, sg, cb, msb_first=msb)
    x = of.round_to(np.random.default_rng(m + d).standard_normal((m, d)).astype(np.float32),
                    "bf16")
    x_rot = of.rpbh_forward_lowp(x, perm.numpy(), sg.numpy(), "bf16")
    bias = of.round_to(np.random.default_rng(n).standard_normal(n).astype(np.float32), "bf16")
    check_linear_lowp(tq, "bf16", x_rot, packed, norms, d, bits, cb, bias, msb)
    order = tq.TQ_MSB_FIRST if msb else tq.TQ_LSB_FIRST
    y = tq.orbit_forward(lp_tensor(x, "bf16").to(DEV), torch.from_numpy(packed).to(DEV),
                         torch.from_numpy(norms).to(DEV), perm.to(DEV), sg.to(DEV), bits, cb,
                         lp_tensor(bias, "bf16").to(DEV), bit_order=order)
    y2 = tq.orbit_linear(lp_tensor(x_rot, "bf16").to(DEV), torch.from_numpy(packed).to(DEV),
                         torch.from_numpy(norms).to(DEV), bits, cb,
                         lp_tensor(bias, "bf16").to(DEV), bit_order=order)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("seed", range(6))
def test_tq3_random_counts(tq, seed):
    """TQ3 round trip at random vector counts and dtypes (every count goes
    through its own grid size; the larger ones reach the pipelined loop)."""
    rng = np.random.default_rng(seed)
    n = int(rng.choice([int(rng.integers(1, 5000)), int(rng.integers(5000, 1 << 18))]))
    dtype = [torch.float32, torch.bfloat16, torch.float16][seed % 3]
    signs = datagen.tq3_signs()
    x = datagen.gaussian_vectors(n, seed=100 + seed)
    xd = x.to(dtype)
    rec = tq.tq3_quantize(xd.to(DEV), signs)
    x32 = xd.to(torch.float32).numpy()
    o_rec = oracle.tq3_quantize(x32, signs.numpy())
    st = compare_tq3_records(rec.reshape(n, 56).cpu().numpy(), o_rec,
                             oracle.tq3_scaled_coeffs(x32, signs.numpy()))
    assert st["exact"], st
    out = tq.tq3_dequantize(rec, signs, dtype=dtype)
    ref = oracle.tq3_dequantize(o_rec, signs.numpy())
    norms = split_records(o_rec)[1]
    assert compare_reconstruction(out.reshape(n, 128), ref, norms, dtype)["exact"]
