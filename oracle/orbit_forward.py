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

For bf16 / fp16 activations the same steps run in the activation's format,
as torch evaluates them on such tensors: every elementwise result (each
butterfly's sum and difference, the final multiply by the fp32 value of
h ** -0.5, the product codebook value times row norm) is formed in fp32 from
operands of that format and rounded to it (round to nearest even); the
codebook and the row norms are first rounded to the format (`.to(dtype)`).
The matmul plus bias is again evaluated in fp64 from those operands; the
product's output rounding to the format belongs to the tolerance.
"""
import numpy as np

from . import orbit_dequantize, rpbh_forward

LOWP = ("bf16", "f16")


def round_to(x, fmt):
    """fp32 values -> the nearest `fmt` value (ties to even), as fp32.
    bf16: keep the upper 16 bits of the fp32 pattern after adding half of the
    dropped part's range (plus the kept part's lowest bit, for ties to even).
    f16: IEEE binary16 through numpy's conversion (round to nearest even)."""
    x = np.asarray(x, dtype=np.float32)
    if fmt == "f16":
        with np.errstate(over="ignore"):  # beyond the format's range: +-inf, as the cast gives
            return x.astype(np.float16).astype(np.float32)
    if fmt != "bf16":
        raise ValueError(fmt)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def fwht_lowp(y, h, fmt):
    """Orthonormal FWHT on each block of h along the last axis of `fmt`
    values: stages of half-width 1, 2, ..., h/2; in each stage element j with
    that bit clear and its partner j + half become round(a + b) and
    round(a - b) (fp32 arithmetic, then rounding to `fmt`); then every value
    becomes round(v * fp32(h ** -0.5))."""
    y = np.array(y, dtype=np.float32)
    d = y.shape[-1]
    j = np.arange(d)
    half = 1
    while half < h:
        lo = j[(j & half) == 0]
        hi = lo + half
        a, b = y[..., lo], y[..., hi]
        y[..., lo] = round_to(a + b, fmt)
        y[..., hi] = round_to(a - b, fmt)
        half *= 2
    return round_to(y * np.float32(h ** -0.5), fmt)


def rpbh_forward_lowp(x, perm, signs, fmt):
    """rpbh_forward on `fmt` activations: gather by perm, times the +-1
    signs (exact), then fwht_lowp with h = d & -d."""
    x = round_to(x, fmt)
    d = x.shape[-1]
    y = x[..., np.asarray(perm, dtype=np.int64)] * np.asarray(signs, dtype=np.float32)
    return fwht_lowp(y, d & -d, fmt)


def orbit_rotated_weight_lowp(packed, norms, d, bits, codebook, fmt, msb_first=True):
    """W' of `fmt`: round(round(codebook[code]) * round(row_norm))."""
    cb = round_to(np.asarray(codebook, dtype=np.float32), fmt)
    from . import unpack
    rows = np.asarray(norms).size
    codes = unpack(np.asarray(packed).reshape(-1), rows * d, bits,
                   msb_first=msb_first).reshape(rows, d)
    nr = round_to(np.asarray(norms, dtype=np.float32).reshape(rows, 1), fmt)
    return round_to(cb[codes] * nr, fmt)


def orbit_forward_lowp(x, packed, norms, perm, signs, bits, codebook, fmt, bias=None,
                       msb_first=True):
    """The forward on `fmt` activations. Returns (x_rot as fp32 values of
    `fmt`, W' likewise, y in fp64 before the output rounding)."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    x_rot = rpbh_forward_lowp(x.reshape(-1, d), perm, signs, fmt)
    w = orbit_rotated_weight_lowp(packed, norms, d, bits, codebook, fmt, msb_first)
    y = x_rot.astype(np.float64) @ w.astype(np.float64).T
    if bias is not None:
        y = y + round_to(np.asarray(bias, dtype=np.float32), fmt).astype(np.float64).reshape(1, -1)
    return x_rot, w, y


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
