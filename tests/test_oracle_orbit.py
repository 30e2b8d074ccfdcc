"""Pins of the oracle's RPBH rotation and OrbitQuant weight codec.

Source: "zerogpu-sdxlTrainer: toolkit/util/orbit_quant.py" -- module docstring
(per-row norms, unit directions, codebook for the N(0, 1/d) marginal, the
runtime identity W' (P x) = W x), hadamard_block_size, rpbh_params, _fwht,
rpbh_forward / rpbh_inverse, pack_codes, _quantize_rows, quantize_,
_dequantize_rotated, dequantize.

Independent references: dense fp64 matrices for the rotation, np.unpackbits
for the page's bit order, and Max (1960)'s Gaussian distortion for quality.
"""
import hashlib
import json
import math
import os

import numpy as np
import pytest

import datagen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def sylvester(n):
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def dense_rotation(d, perm, signs):
    """R = blkdiag(H_h / sqrt(h)) . diag(signs) . P with (P x)_j = x[perm_j]."""
    h = d & -d
    hb = sylvester(h).astype(np.float64) / math.sqrt(h)
    blk = np.kron(np.eye(d // h), hb)
    pm = np.zeros((d, d))
    pm[np.arange(d), np.asarray(perm)] = 1.0
    return blk @ np.diag(np.asarray(signs, dtype=np.float64)) @ pm


def unpack_msb(packed, count, bits):
    stream = np.unpackbits(np.asarray(packed, dtype=np.uint8).reshape(-1), bitorder="big")
    b = stream[: count * bits].reshape(count, bits).astype(np.int64)
    return (b * (1 << np.arange(bits - 1, -1, -1))).sum(1)


def test_block_size():
    import oracle
    for d, h in [(3072, 1024), (4096, 4096), (96, 32), (100, 4), (12288, 4096), (5120, 1024)]:
        assert oracle.block_size(d) == h


def test_rotation_draw_golden():
    with open(os.path.join(GOLDEN, "rpbh_d3072.json")) as f:
        g = json.load(f)
    perm, signs = datagen.rpbh_params(3072)
    assert perm[:8].tolist() == g["perm_head"]
    assert signs[:16].tolist() == g["signs_head"]
    assert hashlib.sha256(perm.numpy().astype("<i8").tobytes()).hexdigest() == g["perm_int64_sha256"]
    assert hashlib.sha256(signs.numpy().astype("i1").tobytes()).hexdigest() == g["signs_int8_sha256"]
    assert sorted(perm.tolist()) == list(range(3072))
    assert set(signs.tolist()) == {-1, 1}


def test_tq3_sign_draw_golden():
    with open(os.path.join(GOLDEN, "tq3_signs.json")) as f:
        g = json.load(f)
    s = datagen.tq3_signs()
    assert hex(int.from_bytes(datagen.sign_mask_bytes(s), "little")) == g["mask_hex"]
    assert int((s > 0).sum()) == g["plus_count"]


@pytest.mark.parametrize("d", [96, 160, 256])
def test_rpbh_matches_dense(oracle_mod, d):
    perm, signs = datagen.rpbh_params(d)
    rng = np.random.default_rng(d)
    w = rng.standard_normal((12, d)).astype(np.float32)
    r = dense_rotation(d, perm.numpy(), signs.numpy())
    y = oracle_mod.rpbh_forward(w, perm, signs)
    ref = w.astype(np.float64) @ r.T
    assert np.max(np.abs(y - ref)) < 1e-5
    back = oracle_mod.rpbh_inverse(y, np.argsort(perm.numpy()), signs)
    assert np.max(np.abs(back - w)) < 1e-5


def test_rpbh_3072_orthogonal(oracle_mod):
    perm, signs = datagen.rpbh_params(3072)
    w = datagen.orbit_weight(rows=8).numpy()
    x = np.random.default_rng(1).standard_normal((8, 3072)).astype(np.float32)
    rw = oracle_mod.rpbh_forward(w, perm, signs).astype(np.float64)
    rx = oracle_mod.rpbh_forward(x, perm, signs).astype(np.float64)
    w64, x64 = w.astype(np.float64), x.astype(np.float64)
    assert np.allclose(np.linalg.norm(rw, axis=1), np.linalg.norm(w64, axis=1), rtol=1e-6)
    assert np.allclose((rw * rx).sum(1), (w64 * x64).sum(1), atol=1e-5)
    back = oracle_mod.rpbh_inverse(rw.astype(np.float32), np.argsort(perm.numpy()), signs)
    assert np.max(np.abs(back - w)) < 1e-7


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [96, 3072])
def test_quantize_matches_fp64_brute_force(oracle_mod, bits, d):
    perm, signs = datagen.rpbh_params(d)
    w = datagen.orbit_weight(rows=16, d=d, seed=40 + bits).numpy()
    cb = oracle_mod.orbit_codebook(bits, d)
    edges = oracle_mod.orbit_edges(cb).astype(np.float64)
    packed, norms = oracle_mod.orbit_quantize(w, bits, perm, signs, cb)
    assert packed.shape == (16, d * bits // 8)
    r = dense_rotation(d, perm.numpy(), signs.numpy())
    y = w.astype(np.float64) @ r.T
    n64 = np.linalg.norm(y, axis=1)
    assert np.max(np.abs(norms - n64) / n64) < 1e-6
    unit = y / n64[:, None]
    want = np.searchsorted(edges, unit, side="left")
    got = unpack_msb(packed, 16 * d, bits).reshape(16, d)
    near = np.min(np.abs(unit[..., None] - edges), axis=-1) < 1e-6 * np.abs(unit).max()
    assert np.array_equal(got[~near], want[~near])
    assert near.mean() < 1e-3
    # the LSB-first layout carries the same codes
    pl, nl = oracle_mod.orbit_quantize(w, bits, perm, signs, cb, msb_first=False)
    assert np.array_equal(nl, norms)
    lsb = np.unpackbits(pl.reshape(-1), bitorder="little")[: 16 * d * bits]
    codes_l = (lsb.reshape(-1, bits).astype(np.int64) * (1 << np.arange(bits))).sum(1)
    assert np.array_equal(codes_l, got.reshape(-1))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_dequantize_matches_fp64(oracle_mod, bits):
    d = 3072
    perm, signs = datagen.rpbh_params(d)
    inv = np.argsort(perm.numpy())
    w = datagen.orbit_weight(rows=6, d=d, seed=50).numpy()
    cb = oracle_mod.orbit_codebook(bits, d)
    packed, norms = oracle_mod.orbit_quantize(w, bits, perm, signs, cb)
    codes = unpack_msb(packed, 6 * d, bits).reshape(6, d)
    rot = oracle_mod.orbit_dequantize(packed, norms, d, bits, inv, signs, cb,
                                      rotated_only=True)
    assert np.max(np.abs(rot - cb[codes].astype(np.float64) * norms[:, None])) \
        <= 1e-7 * norms.max()
    full = oracle_mod.orbit_dequantize(packed, norms, d, bits, inv, signs, cb)
    r = dense_rotation(d, perm.numpy(), signs.numpy())
    ref = rot.astype(np.float64) @ r          # R^T applied to each row
    assert np.max(np.abs(full - ref)) < 1e-6 * norms.max()
    # the runtime identity: W' (R x) == W_hat x
    x = np.random.default_rng(2).standard_normal((3, d)).astype(np.float64)
    assert np.allclose(rot.astype(np.float64) @ (r @ x.T), full.astype(np.float64) @ x.T,
                       atol=1e-5 * norms.max())


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quality_matches_gaussian_distortion(oracle_mod, bits):
    # Rotated unit-row coordinates are close to N(0, 1/d), so the relative
    # squared error approaches the Gaussian quantiser's distortion (Max 1960:
    # 0.1175, 0.03454, 0.009497 for 4, 8, 16 levels).
    mse = {2: 0.1175, 3: 0.03454, 4: 0.009497}[bits]
    d = 3072
    perm, signs = datagen.rpbh_params(d)
    w = datagen.orbit_weight(rows=128).numpy()
    cb = oracle_mod.orbit_codebook(bits, d)
    packed, norms = oracle_mod.orbit_quantize(w, bits, perm, signs, cb)
    full = oracle_mod.orbit_dequantize(packed, norms, d, bits, np.argsort(perm.numpy()),
                                       signs, cb)
    rel = np.linalg.norm(full - w) / np.linalg.norm(w)
    assert abs(rel - math.sqrt(mse)) < 0.03 * math.sqrt(mse)


# ---- rows longer than 4096: Hadamard blocks of up to 16384 ---------------

def sylvester_rotate_fp64(w, perm, signs):
    """Rows of R w for R = blkdiag(H_h / sqrt(h)) . diag(signs) . P in fp64,
    with the Sylvester matrix's closed form H[i, j] = (-1)^popcount(i & j)
    evaluated directly (no staged transform), 1024 outputs at a time."""
    w = np.asarray(w, dtype=np.float64)
    d = w.shape[1]
    h = d & -d
    v = w[:, np.asarray(perm)] * np.asarray(signs, dtype=np.float64)[None, :]
    out = np.empty_like(v)
    j = np.arange(h, dtype=np.uint32)[None, :]
    step = min(h, 1024)
    for i0 in range(0, h, step):
        i = np.arange(i0, i0 + step, dtype=np.uint32)[:, None]
        sg = 1.0 - 2.0 * (np.bitwise_count(i & j) & 1)          # [step, h]
        for b in range(d // h):
            out[:, b * h + i0: b * h + i0 + step] = v[:, b * h:(b + 1) * h] @ sg.T
    return out / math.sqrt(h)


_LARGE_D = {}


def _large_case(d):
    """Two weight rows of width d and their fp64 rotation (cached per d)."""
    if d not in _LARGE_D:
        perm, signs = datagen.rpbh_params(d)
        w = datagen.orbit_weight(rows=2, d=d, seed=d + 7).numpy()
        _LARGE_D[d] = (perm, signs, w, sylvester_rotate_fp64(w, perm.numpy(), signs.numpy()))
    return _LARGE_D[d]


def test_sylvester_closed_form_is_the_dense_matrix():
    # the closed form reproduces the recursive construction (so it can stand
    # in for a dense matrix too large to build at d = 16384)
    for n in (32, 256):
        i = np.arange(n, dtype=np.uint32)
        cf = 1 - 2 * (np.bitwise_count(i[:, None] & i[None, :]) & 1).astype(np.int64)
        assert np.array_equal(cf, sylvester(n))


@pytest.mark.parametrize("d", [5120, 8192, 12288, 16384])
def test_rpbh_large_d_matches_closed_form(oracle_mod, d):
    perm, signs, w, ref = _large_case(d)
    assert oracle_mod.block_size(d) == (d & -d)
    y = oracle_mod.rpbh_forward(w, perm, signs).astype(np.float64)
    nrm = np.linalg.norm(w.astype(np.float64), axis=1)
    assert np.max(np.abs(y - ref) / nrm[:, None]) < 2e-6
    assert np.allclose(np.linalg.norm(y, axis=1), nrm, rtol=1e-6)
    back = oracle_mod.rpbh_inverse(y.astype(np.float32), np.argsort(perm.numpy()), signs)
    assert np.max(np.abs(back - w) / nrm[:, None]) < 2e-6


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [12288, 16384])
def test_quantize_large_d_matches_fp64(oracle_mod, bits, d):
    perm, signs, w, y = _large_case(d)
    cb = oracle_mod.orbit_codebook(bits, d)
    edges = oracle_mod.orbit_edges(cb).astype(np.float64)
    packed, norms = oracle_mod.orbit_quantize(w, bits, perm, signs, cb)
    n64 = np.linalg.norm(y, axis=1)
    assert np.max(np.abs(norms - n64) / n64) < 1e-6
    unit = y / n64[:, None]
    want = np.searchsorted(edges, unit, side="left")
    got = unpack_msb(packed, 2 * d, bits).reshape(2, d)
    near = np.min(np.abs(unit[..., None] - edges), axis=-1) < 1e-6 * np.abs(unit).max()
    assert np.array_equal(got[~near], want[~near])
    assert near.mean() < 1e-3
