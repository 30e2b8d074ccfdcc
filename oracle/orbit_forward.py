"""Oracle for the OrbitQuant runtime forward (a linear layer with a quantized weight).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "zerogpu-sdxlTrainer: toolkit/util/orbit_quant.py", the module
docstring (the forward rotation is applied to the activations instead of
un-rotating the weight, so the two cancel in the matmul) and
OrbitQuantizer.forward: the rotated-basis weight W' = _dequantize_rotated
(codebook value times row norm, in the activation dtype), x_rot =
rpbh_forward(x), y = F.linear(x_rot, W', bias).

The oracle follows those steps for fp32 activations: x_rot and W' come from
the C oracle in fp32 with the page's operation order (they are fixed bit for
bit), and the matmul plus bias is evaluated in fp64 (the page leaves its
summation order to the BLAS).
"""
import numpy as np

from . import orbit_dequantize, rpbh_forward


def orbit_rotated_weight(packed, norms, d, bits, codebook, msb_first=True):
    """W' [rows, d] fp32: codebook[code] * row_norm, as _dequantize_rotated."""
    dummy_perm = np.arange(d, dtype=np.int64)
    dummy_signs = np.ones(d, dtype=np.int8)
    return orbit_dequantize(packed, norms, d, bits, dummy_perm, dummy_signs, codebook,
                            msb_first=msb_first, rotated_only=True)


def orbit_linear(x_rot, packed, norms, d, bits, codebook, bias=None, msb_first=True):
    """y = x_rot @ W'^T (+ bias) in fp64 from the fp32 operands."""
    w = orbit_rotated_weight(packed, norms, d, bits, codebook, msb_first).astype(np.float64)
    y = np.asarray(x_rot, dtype=np.float64).reshape(-1, d) @ w.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64).reshape(1, -1)
    return y


def orbit_forward(x, packed, norms, perm, signs, bits, codebook, bias=None, msb_first=True):
    """The whole forward: rpbh_forward(x) (fp32, the page's order), then the
    linear layer with the rotated-basis weight. Returns (x_rot fp32, y fp64)."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    x_rot = rpbh_forward(x.reshape(-1, d), perm, signs)
    return x_rot, orbit_linear(x_rot, packed, norms, d, bits, codebook, bias, msb_first)
