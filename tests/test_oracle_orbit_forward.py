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


# ----------------------------------------------- bf16 / fp16 activations ---

import torch  # noqa: E402
from scipy.linalg import hadamard  # noqa: E402


@pytest.mark.parametrize("fmt,tdt", [("bf16", torch.bfloat16), ("f16", torch.float16)])
def test_round_to_matches_torch_conversion(fmt, tdt):
    """The rounding to the narrow format is torch's own fp32 -> dtype cast
    (round to nearest even), including exact ties and values near the top."""
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 50,
                        np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -11, 1 + 3 * 2 ** -11,
                                    -(1 + 2 ** -8), 0.0, -0.0, 257.0, 65504.0, 3e38])])
    want = torch.from_numpy(x).to(tdt).to(torch.float32).numpy()
    got = of.round_to(x, fmt)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_fwht_lowp_rounds_every_stage():
    """Worked by hand, h = 4, x = (256, 1, 1, 0). bf16 has 8 significant
    bits, so 257 is a tie between 256 and 258 and goes to the even 256:
    stage 1 gives (256, 255, 1, 1), stage 2 (256, 256, 255, 254), times 0.5
    (128, 128, 127.5, 127). In fp16 every intermediate is exact:
    (258, 256, 256, 254) / 2."""
    x = np.float32([256, 1, 1, 0])
    assert np.array_equal(of.fwht_lowp(x, 4, "bf16"), np.float32([128, 128, 127.5, 127]))
    assert np.array_equal(of.fwht_lowp(x, 4, "f16"), np.float32([129, 128, 128, 127]))


@pytest.mark.parametrize("d,fmt,bound", [(96, "bf16", 2), (192, "bf16", 2), (96, "f16", 2),
                                          (256, "f16", 1), (1536, "f16", 1)])
def test_rpbh_lowp_on_small_integers_is_one_rounding(d, fmt, bound):
    """Integer inputs in [-bound, bound]: every partial sum is an integer of
    magnitude <= bound * h, exact in the format (<= 256 in bf16, <= 2048 in
    fp16), so the only rounding left is the final scaling: the result is the
    dense Hadamard product (scipy's Sylvester matrix) of the gathered, signed
    row times fp32(h ** -0.5), rounded once."""
    h = d & -d
    assert bound * h <= (256 if fmt == "bf16" else 2048)
    rng = np.random.default_rng(d)
    x = rng.integers(-bound, bound + 1, size=(5, d)).astype(np.float32)
    perm, sg = datagen.rpbh_params(d)
    perm, sg = perm.numpy(), sg.numpy().astype(np.float32)
    y = x[:, perm] * sg
    H = hadamard(h).astype(np.float64)
    dense = (y.reshape(5, d // h, h).astype(np.float64) @ H.T).reshape(5, d)
    want = of.round_to(dense.astype(np.float32) * np.float32(h ** -0.5), fmt)
    assert np.array_equal(of.rpbh_forward_lowp(x, perm, sg, fmt), want)


def test_rotated_weight_lowp_worked_example():
    """0.1 and 3.0 as codebook value and row norm. bf16: 0.1 -> 0.10009765625,
    times 3 = 0.30029296875 = 153.75 ulps of 2^-9 -> 154 ulps = 0.30078125.
    fp16: 0.1 -> 0.0999755859375, times 3 = 0.2999267578125 = 1228.5 ulps of
    2^-12, a tie -> 1228 ulps = 0.2998046875."""
    packed = oracle.pack(np.zeros(32, dtype=np.uint8), 2, msb_first=True)
    cb = np.float32([0.1, 0.2, 0.3, 0.4])
    wb = of.orbit_rotated_weight_lowp(packed, np.float32([3.0]), 32, 2, cb, "bf16")
    wh = of.orbit_rotated_weight_lowp(packed, np.float32([3.0]), 32, 2, cb, "f16")
    assert np.all(wb == np.float32(0.30078125)) and np.all(wh == np.float32(0.2998046875))


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_forward_lowp_zero_input_and_fp32_agreement(fmt):
    """Zero input gives the rounded bias exactly; otherwise the narrow forward
    stays within its rounding budget of the fp32 forward (each of the log2(h)
    stages, the scaling and W' add at most one unit roundoff of the format)."""
    d, bits = 768, 3
    w, perm, sg, cb, packed, norms = quantized(48, d, bits, 31)
    bias = np.random.default_rng(4).standard_normal(48).astype(np.float32)
    _, _, y0 = of.orbit_forward_lowp(np.zeros((2, d), np.float32), packed, norms, perm, sg, bits,
                                     cb, fmt, bias)
    assert np.array_equal(y0, np.broadcast_to(of.round_to(bias, fmt).astype(np.float64), y0.shape))
    x = of.round_to(np.random.default_rng(5).standard_normal((8, d)).astype(np.float32), fmt)
    _, _, y = of.orbit_forward_lowp(x, packed, norms, perm, sg, bits, cb, fmt)
    _, y32 = of.orbit_forward(x, packed, norms, perm, sg, bits, cb)
    u = 2.0 ** -8 if fmt == "bf16" else 2.0 ** -11
    stages = int(np.log2(d & -d)) + 3
    scale = np.abs(x).astype(np.float64) @ np.abs(of.orbit_rotated_weight(packed, norms, d, bits, cb)).T
    # the rotation's growth: each stage's error enters every later sum
    assert np.all(np.abs(y - y32) <= stages * u * np.sqrt(d) * scale + 1e-12)
