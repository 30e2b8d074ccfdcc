"""Plain, slow, obviously-correct CPU oracle for the TQ3 and OrbitQuant codecs.

TEST INFRASTRUCTURE ONLY. Only tests/, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` import this package. The product package
(randomized_hadamard_lloyd_amd) never imports it and shares no code with it.

The arithmetic lives in ``tq_oracle.c`` (IEEE fp32, declared operation order)
and ``lloyd_max.py`` (fp64 codebook procedure). This module only marshals numpy
arrays into the C functions.

Pins (what fixes each function independently of itself) are in
tests/test_oracle_*.py. Parity status per function:
  * TQ3 quantize / dequantize, FWHT, packing: pinned.
  * Gaussian Lloyd-Max: pinned (textbook tables, fixed-point conditions).
  * RPBH forward / inverse: pinned (dense-matrix brute force, orthogonality).
  * OrbitQuant quantize / dequantize: pinned against brute force on small
    rows; reconstruction quality on the config-5 weights is parity unpinned
    (the page prints no figure for it).
  * OrbitQuant forward (orbit_forward.py): pinned by the cancellation of the
    two rotations, the zero input, an independent unpack of the rotated
    weight, and the distortion against the unquantized layer. Its bf16 /
    fp16 form is pinned by torch's own casts (the rounding), a hand-worked
    per-stage rounding case, the dense Hadamard product on integer inputs
    (one rounding), a hand-worked W' product, and the zero input.
  * Decode attention over TQ3 records (attention.py): pinned by closed forms
    (one token, zero scale, duplicate keys, a dominant key) and invariants
    (token order, query-head grouping).
"""
import ctypes
import os

import numpy as np

from .lloyd_max import (gaussian_lloyd_max, gaussian_lloyd_max_f64,  # noqa: F401
                        orbit_codebook, orbit_edges)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_f32p = ctypes.POINTER(ctypes.c_float)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i8p = ctypes.POINTER(ctypes.c_int8)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64
_int = ctypes.c_int


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    sigs = {
        "orc_fwht": [_f32p, _i64, _int],
        "orc_fwht_orbit": [_f32p, _i64, _int],
        "orc_pack_lsb": [_u8p, _i64, _int, _u8p],
        "orc_unpack_lsb": [_u8p, _i64, _int, _u8p],
        "orc_pack_msb": [_u8p, _i64, _int, _u8p],
        "orc_unpack_msb": [_u8p, _i64, _int, _u8p],
        "orc_tq3_quantize": [_f32p, _i64, _f32p, _int, _u8p, _int],
        "orc_tq3_dequantize": [_u8p, _i64, _f32p, _int, _f32p, _int],
        "orc_tq3_scaled_coeffs": [_f32p, _i64, _f32p, _f32p, _int],
        "orc_rpbh_forward": [_f32p, _i64, _i64, _i64p, _i8p, _f32p, _int],
        "orc_rpbh_inverse": [_f32p, _i64, _i64, _i64p, _i8p, _f32p, _int],
        "orc_orbit_quantize": [_f32p, _i64, _i64, _int, _i64p, _i8p, _f32p,
                               _int, _u8p, _f32p, _int],
        "orc_orbit_dequantize": [_u8p, _f32p, _i64, _i64, _int, _i64p, _i8p,
                                 _f32p, _int, _int, _f32p, _int],
        "orc_orbit_unit": [_f32p, _i64, _i64, _i64p, _i8p, _f32p, _f32p, _int],
        "orc_tq3_bucketize": [_f32p, _i64, _u8p],
        "orc_tq3_tables": [_f32p, _f32p],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = None
    lib.orc_block_size.argtypes = [_i64]
    lib.orc_block_size.restype = _i64
    lib.orc_max_threads.argtypes = []
    lib.orc_max_threads.restype = _int
    _lib = lib
    return lib


def _np(a, dtype):
    """Contiguous numpy copy/view of a numpy array or CPU torch tensor."""
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def max_threads() -> int:
    return _load().orc_max_threads()


# ------------------------------------------------------------------ TQ3 ---

def tq3_quantize(x, signs, post_flip=False, threads=0):
    """x: [n, 128] float (upcast to fp32 exactly); signs: [128] of +-1.
    Returns uint8 [n, 56] records: 48 bytes of LSB-first 3-bit indices, the
    fp32 norm, the fp32 scale."""
    lib = _load()
    x = _np(x, np.float32).reshape(-1, 128)
    s = _np(signs, np.float32).reshape(128)
    rec = np.zeros((x.shape[0], 56), dtype=np.uint8)
    lib.orc_tq3_quantize(_p(x, ctypes.c_float), x.shape[0], _p(s, ctypes.c_float),
                         int(bool(post_flip)), _p(rec, ctypes.c_uint8), threads)
    return rec


def tq3_dequantize(rec, signs, post_flip=False, threads=0):
    """rec: uint8 [n, 56] -> fp32 [n, 128]."""
    lib = _load()
    rec = _np(rec, np.uint8).reshape(-1, 56)
    s = _np(signs, np.float32).reshape(128)
    y = np.zeros((rec.shape[0], 128), dtype=np.float32)
    lib.orc_tq3_dequantize(_p(rec, ctypes.c_uint8), rec.shape[0],
                           _p(s, ctypes.c_float), int(bool(post_flip)),
                           _p(y, ctypes.c_float), threads)
    return y


def tq3_scaled_coeffs(x, signs, threads=0):
    """Per-coefficient value divided by the vector's scale, just before the
    codebook lookup: fp32 [n, 128]."""
    lib = _load()
    x = _np(x, np.float32).reshape(-1, 128)
    s = _np(signs, np.float32).reshape(128)
    xs = np.zeros_like(x)
    lib.orc_tq3_scaled_coeffs(_p(x, ctypes.c_float), x.shape[0],
                              _p(s, ctypes.c_float), _p(xs, ctypes.c_float), threads)
    return xs


def tq3_bucketize(xs):
    """Codebook index (0..7) of each given normalised value."""
    lib = _load()
    xs = _np(xs, np.float32).reshape(-1)
    out = np.zeros(xs.shape, dtype=np.uint8)
    lib.orc_tq3_bucketize(_p(xs, ctypes.c_float), xs.size, _p(out, ctypes.c_uint8))
    return out


def tq3_tables():
    """(centroids [8], boundaries [7]) as fp32, as the oracle holds them."""
    lib = _load()
    c = np.zeros(8, dtype=np.float32)
    b = np.zeros(7, dtype=np.float32)
    lib.orc_tq3_tables(_p(c, ctypes.c_float), _p(b, ctypes.c_float))
    return c, b


def tq3_split(rec):
    """(packed [n,48] u8, norms [n] f32, scales [n] f32) views of records."""
    rec = _np(rec, np.uint8).reshape(-1, 56)
    norms = rec[:, 48:52].copy().view(np.float32).reshape(-1)
    scales = rec[:, 52:56].copy().view(np.float32).reshape(-1)
    return rec[:, :48], norms, scales


def fwht(x, normalize="tq3"):
    """Normalised FWHT along the last axis (power-of-two length)."""
    lib = _load()
    x = _np(x, np.float32).copy()
    n = x.shape[-1]
    fn = lib.orc_fwht if normalize == "tq3" else lib.orc_fwht_orbit
    fn(_p(x, ctypes.c_float), x.size // n, n)
    return x


def pack(codes, bits, msb_first=False):
    lib = _load()
    c = _np(codes, np.uint8).reshape(-1)
    out = np.zeros(((c.size * bits + 7) // 8,), dtype=np.uint8)
    fn = lib.orc_pack_msb if msb_first else lib.orc_pack_lsb
    fn(_p(c, ctypes.c_uint8), c.size, bits, _p(out, ctypes.c_uint8))
    return out


def unpack(packed, count, bits, msb_first=False):
    lib = _load()
    p = _np(packed, np.uint8).reshape(-1)
    assert p.size * 8 >= count * bits
    out = np.zeros((count,), dtype=np.uint8)
    fn = lib.orc_unpack_msb if msb_first else lib.orc_unpack_lsb
    fn(_p(p, ctypes.c_uint8), count, bits, _p(out, ctypes.c_uint8))
    return out


# ----------------------------------------------------------- OrbitQuant ---

def block_size(d: int) -> int:
    return int(_load().orc_block_size(d))


def _check_orbit(d):
    h = d & (-d)
    if h < 8 or h > 65536:
        raise ValueError(f"oracle supports Hadamard blocks 8..65536, got {h}")


def rpbh_forward(w, perm, signs, threads=0):
    lib = _load()
    w = _np(w, np.float32)
    rows, d = w.reshape(-1, w.shape[-1]).shape
    _check_orbit(d)
    pm = _np(perm, np.int64)
    sg = _np(signs, np.int8)
    y = np.zeros((rows, d), dtype=np.float32)
    lib.orc_rpbh_forward(_p(w, ctypes.c_float), rows, d, _p(pm, ctypes.c_int64),
                         _p(sg, ctypes.c_int8), _p(y, ctypes.c_float), threads)
    return y


def rpbh_inverse(y, inv_perm, signs, threads=0):
    lib = _load()
    y = _np(y, np.float32)
    rows, d = y.reshape(-1, y.shape[-1]).shape
    _check_orbit(d)
    ip = _np(inv_perm, np.int64)
    sg = _np(signs, np.int8)
    out = np.zeros((rows, d), dtype=np.float32)
    lib.orc_rpbh_inverse(_p(y, ctypes.c_float), rows, d, _p(ip, ctypes.c_int64),
                         _p(sg, ctypes.c_int8), _p(out, ctypes.c_float), threads)
    return out


def orbit_quantize(w, bits, perm, signs, codebook, msb_first=True, threads=0):
    """Returns (packed uint8 [rows, d*bits/8], row_norms fp32 [rows])."""
    lib = _load()
    w = _np(w, np.float32)
    rows, d = w.shape
    _check_orbit(d)
    pm = _np(perm, np.int64)
    sg = _np(signs, np.int8)
    cb = _np(codebook, np.float32)
    assert cb.size == 2 ** bits
    packed = np.zeros((rows, d * bits // 8), dtype=np.uint8)
    norms = np.zeros((rows,), dtype=np.float32)
    lib.orc_orbit_quantize(_p(w, ctypes.c_float), rows, d, bits,
                           _p(pm, ctypes.c_int64), _p(sg, ctypes.c_int8),
                           _p(cb, ctypes.c_float), int(bool(msb_first)),
                           _p(packed, ctypes.c_uint8), _p(norms, ctypes.c_float),
                           threads)
    return packed, norms


def orbit_dequantize(packed, norms, d, bits, inv_perm, signs, codebook,
                     msb_first=True, rotated_only=False, threads=0):
    lib = _load()
    _check_orbit(d)
    pk = _np(packed, np.uint8)
    nr = _np(norms, np.float32).reshape(-1)
    rows = nr.size
    assert pk.size == rows * d * bits // 8
    ip = _np(inv_perm, np.int64)
    sg = _np(signs, np.int8)
    cb = _np(codebook, np.float32)
    out = np.zeros((rows, d), dtype=np.float32)
    lib.orc_orbit_dequantize(_p(pk, ctypes.c_uint8), _p(nr, ctypes.c_float), rows,
                             d, bits, _p(ip, ctypes.c_int64), _p(sg, ctypes.c_int8),
                             _p(cb, ctypes.c_float), int(bool(msb_first)),
                             int(bool(rotated_only)), _p(out, ctypes.c_float),
                             threads)
    return out


def orbit_unit(w, perm, signs, threads=0):
    """(unit directions fp32 [rows, d], row norms fp32 [rows]) before bucketing."""
    lib = _load()
    w = _np(w, np.float32)
    rows, d = w.shape
    _check_orbit(d)
    pm = _np(perm, np.int64)
    sg = _np(signs, np.int8)
    unit = np.zeros((rows, d), dtype=np.float32)
    norms = np.zeros((rows,), dtype=np.float32)
    lib.orc_orbit_unit(_p(w, ctypes.c_float), rows, d, _p(pm, ctypes.c_int64),
                       _p(sg, ctypes.c_int8), _p(unit, ctypes.c_float),
                       _p(norms, ctypes.c_float), threads)
    return unit, norms
