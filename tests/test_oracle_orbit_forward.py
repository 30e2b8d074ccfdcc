"""Pins of the OrbitQuant-forward oracle (oracle/orbit_forward.py).

Source: "zerogpu-sdxlTrainer: toolkit/util/orbit_quant.py": the module
docstring (rotating the activation instead of un-rotating the weight; the two
rotations cancel in the matmul) and OrbitQuantizer.forward. The pins check
the forward against routes that do not share its composition: the fully
dequantized weight applied to the unrotated input, the zero input, and the
original weight's product within the quantizer's distortion.
"""
import numpy as np
import pytest

import datagen
import oracle
from oracle import orbit_forward as of


def quantized(rows, d, bits, seed):
    w = np.random.default_rng(seed).standard_normal((rows, d)).astype(np.float32) * 0.02
    perm, sg = datagen.rpbh_params(d)
    cb = oracle.orbit_codebook(bits, d)
    packed, norms = oracle.orbit_quantize(w, bits, perm, sg, cb)
    return w, perm.numpy(), sg.numpy(), cb, packed, norms


@pytest.mark.parametrize("d,bits", [(96, 2), (512, 3), (3072, 4), (1536, 3)])
def test_rotations_cancel(d, bits):
    """rpbh_forward(x) W'^T equals x W_hat^T, W_hat = dequantize(full) =
    rpbh_inverse(W'): the forward rotation is the transpose of the inverse."""
    w, perm, sg, cb, packed, norms = quantized(40, d, bits, d + bits)
    x = np.random.default_rng(7).standard_normal((9, d)).astype(np.float32)
    _, y = of.orbit_forward(x, packed, norms, perm, sg, bits, cb)
    inv = np.argsort(perm)
    w_hat = oracle.orbit_dequantize(packed, norms, d, bits, inv, sg, cb).astype(np.float64)
    y2 = x.astype(np.float64) @ w_hat.T
    scale = np.abs(x).astype(np.float64) @ np.abs(w_hat).T
    assert np.all(np.abs(y - y2) <= 64 * 2.0 ** -24 * scale + 1e-12)


def test_zero_input_gives_bias():
    w, perm, sg, cb, packed, norms = quantized(24, 256, 3, 1)
    bias = np.random.default_rng(2).standard_normal(24).astype(np.float32)
    _, y = of.orbit_forward(np.zeros((3, 256), np.float32), packed, norms, perm, sg, 3, cb, bias)
    assert np.array_equal(y, np.broadcast_to(bias.astype(np.float64), y.shape))


def test_rotated_weight_is_codebook_times_norm():
    """W' entries are the codebook values of the unpacked codes times the row
    norm (fp32 products), by an independent unpack of the MSB-first stream."""
    d, bits = 128, 3
    w, perm, sg, cb, packed, norms = quantized(5, d, bits, 3)
    wr = of.orbit_rotated_weight(packed, norms, d, bits, cb)
    codes = oracle.unpack(packed.reshape(-1), 5 * d, bits, msb_first=True).reshape(5, d)
    expect = (cb[codes].astype(np.float32) * norms[:, None].astype(np.float32)).astype(np.float32)
    assert np.array_equal(wr, expect)


@pytest.mark.parametrize("bits,min_cos", [(2, 0.90), (3, 0.97), (4, 0.99)])
def test_forward_tracks_the_unquantized_layer(bits, min_cos):
    """y approximates x W^T with the codebook's distortion (Gaussian weights)."""
    w, perm, sg, cb, packed, norms = quantized(256, 1024, bits, 10 + bits)
    x = np.random.default_rng(11).standard_normal((16, 1024)).astype(np.float32)
    _, y = of.orbit_forward(x, packed, norms, perm, sg, bits, cb)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    cos = (y * ref).sum() / np.sqrt((y * y).sum() * (ref * ref).sum())
    assert cos > min_cos
