"""Pins of the oracle's TQ3 codec against things other than itself.

Source: "ComfyUI-TurboQuant: tq3_core.py" -- module docstring (format and
algorithm steps 1-6, the sign-before-transform argument), the codebook and
boundary tables, tq3_quantize / tq3_dequantize, tq3_memory_bytes, the
self-test cases [1], [2], [5], [6], and the change note's measurement of the
broken order (constant block: cosine 0.611, relative L2 error 1.27).
"""
import math

import numpy as np
import pytest

import datagen


def sylvester(n):
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


H128 = sylvester(128).astype(np.float64)


def page_group_unpack(packed):
    """The page's _unpack_3bit formulation (24-bit little-endian words)."""
    p = np.asarray(packed, dtype=np.int64).reshape(-1, 48)
    idx = np.zeros((p.shape[0], 128), dtype=np.int64)
    for g in range(16):
        word = p[:, 3 * g] | (p[:, 3 * g + 1] << 8) | (p[:, 3 * g + 2] << 16)
        for i in range(8):
            idx[:, 8 * g + i] = (word >> (3 * i)) & 7
    return idx


def fp64_quantize_chain(x, s):
    """Steps 1-4 evaluated in float64 with a dense Hadamard matrix."""
    x = np.asarray(x, dtype=np.float64)
    n = np.maximum(np.linalg.norm(x, axis=1), 1e-8)
    u = x / n[:, None] * np.asarray(s, dtype=np.float64)[None, :]
    y = u @ H128.T / math.sqrt(128.0)
    scale = np.maximum(np.abs(y).max(axis=1), 1e-8)
    return n, scale, y / scale[:, None]


def cosine_rows(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return (a * b).sum(1) / (np.linalg.norm(a, axis=1) * np.linalg.norm(b, axis=1))


@pytest.fixture(scope="module")
def signs():
    return datagen.tq3_signs().numpy()


# ------------------------------------------------------------- tables ---

def test_tables_nearest_neighbour_condition(oracle_mod):
    # A Lloyd-Max codebook's boundaries are midpoints of neighbouring
    # centroids; the printed table satisfies this to its 4 printed decimals.
    c, b = oracle_mod.tq3_tables()
    mids = (c[:-1].astype(np.float64) + c[1:]) / 2
    assert np.all(np.abs(mids - b) <= 0.5e-4 + 1e-7)
    assert np.array_equal(c, -c[::-1]) and np.array_equal(b, -b[::-1])
    assert np.all(np.diff(c) > 0) and np.all(np.diff(b) > 0)
    assert np.all((b > c[:-1]) & (b < c[1:]))


# ------------------------------------------------------------ bucketing ---

def test_bucket_tie_table(oracle_mod):
    # searchsorted with the default left side: a value equal to a boundary
    # falls in the lower cell, on both signs; -0.0 compares equal to 0.0
    vals = np.array([0.0, -0.0, 0.2304, -0.2304, 0.4824, -0.4824, 0.7992,
                     -0.7992, 1.0, -1.0], dtype=np.float32)
    want = [3, 3, 4, 2, 5, 1, 6, 0, 7, 0]
    assert oracle_mod.tq3_bucketize(vals).tolist() == want


def test_bucket_equals_library_searchsorted(oracle_mod):
    _, b = oracle_mod.tq3_tables()
    rng = np.random.default_rng(11)
    xs = np.concatenate([rng.uniform(-1, 1, 200000).astype(np.float32), b,
                         np.nextafter(b, np.float32(2)), np.nextafter(b, np.float32(-2))])
    assert np.array_equal(oracle_mod.tq3_bucketize(xs),
                          np.searchsorted(b, xs, side="left").astype(np.uint8))


# ------------------------------------------------ brute-force fp64 chain ---

def test_quantize_matches_fp64_chain(oracle_mod, signs):
    x = datagen.gaussian_vectors(512, seed=21).numpy()
    x[:8] = 2.5                                   # constant rows too
    rec = oracle_mod.tq3_quantize(x, signs)
    packed, norms, scales = oracle_mod.tq3_split(rec)
    n64, s64, xs64 = fp64_quantize_chain(x, signs)
    assert np.max(np.abs(norms - n64) / n64) < 1e-6
    assert np.max(np.abs(scales - s64) / s64) < 1e-6
    xs32 = oracle_mod.tq3_scaled_coeffs(x, signs)
    assert np.max(np.abs(xs32 - xs64)) < 2e-6
    _, b = oracle_mod.tq3_tables()
    idx64 = np.searchsorted(b.astype(np.float64), xs64, side="left")
    idx = page_group_unpack(packed)
    near = np.min(np.abs(xs64[..., None] - b.astype(np.float64)), axis=-1) < 2e-6
    assert np.array_equal(idx[~near], idx64[~near])
    assert near.sum() <= 8 * 128 // 4 + 10   # ties: the constant rows' zeros


def test_dequantize_matches_fp64(oracle_mod, signs):
    rec = datagen.decode_records(256, seed=9).numpy()
    y = oracle_mod.tq3_dequantize(rec, signs)
    packed, norms, scales = oracle_mod.tq3_split(rec)
    c, _ = oracle_mod.tq3_tables()
    coef = c[page_group_unpack(packed)].astype(np.float64) * scales[:, None]
    ref = (coef @ H128.T / math.sqrt(128.0)) * signs[None, :] * norms[:, None]
    assert np.max(np.abs(y - ref) / norms[:, None]) < 1e-6


# ------------------------------------------------ the page's self-tests ---

def _round_trip(oracle_mod, x, signs, post_flip=False):
    rec = oracle_mod.tq3_quantize(x, signs, post_flip=post_flip)
    return oracle_mod.tq3_dequantize(rec, signs, post_flip=post_flip)


def test_self_test_single_block(oracle_mod, signs):
    x = datagen.gaussian_vectors(1, seed=123).numpy()
    assert cosine_rows(x, _round_trip(oracle_mod, x, signs)).mean() > 0.97


def test_self_test_batch_and_ratio(oracle_mod, signs):
    # (4, 32, 512): four 128-blocks per row; cosine taken over 512-rows
    x = datagen.gaussian_vectors(4 * 32 * 4, seed=124).numpy()
    xr = _round_trip(oracle_mod, x, signs)
    cos = cosine_rows(x.reshape(-1, 512), xr.reshape(-1, 512)).mean()
    assert cos > 0.97
    numel = 4 * 32 * 512
    compressed, fp16 = (numel // 128) * 56, numel * 2
    assert fp16 / compressed > 4.0 and abs(fp16 / compressed - 256 / 56) < 1e-12


def test_ltx_kv_estimate_sizes():
    # self-test [5]: (2, 64, 64, 2048, 128) -> sizes from the page's formula
    numel = 2 * 64 * 64 * 2048 * 128
    assert numel * 2 == 4_294_967_296
    assert numel // 128 * 56 == 939_524_096


def test_self_test_structured_blocks(oracle_mod, signs):
    rng = np.random.default_rng(6)
    ramp = np.linspace(0.0, 2 * math.pi, 128, dtype=np.float32)
    cases = {
        "constant": np.full((16, 128), 2.5, dtype=np.float32),
        "gaussian + DC offset": (rng.standard_normal((16, 128)) + 3.0).astype(np.float32),
        "low-frequency": np.stack([np.sin(ramp * np.float32(1 + i * 0.1))
                                   for i in range(16)]).astype(np.float32),
        "outlier channel": rng.standard_normal((16, 128)).astype(np.float32),
    }
    cases["outlier channel"][:, 7] = 40.0
    for name, x in cases.items():
        cos = cosine_rows(x, _round_trip(oracle_mod, x, signs)).mean()
        assert cos > 0.97, (name, cos)


def test_gaussian_workload_quality(oracle_mod, signs):
    x = datagen.gaussian_vectors().numpy()
    cos = cosine_rows(x, _round_trip(oracle_mod, x, signs))
    assert cos.mean() > 0.97
    assert 0.975 < cos.mean() < 0.985


# ---------------------------------------- sign flips before the FWHT ---

def test_broken_order_constant_block_closed_form(oracle_mod, signs):
    # Flipping after the transform leaves a constant block as one Hadamard
    # coefficient of +-1 and 127 exact zeros (index 3, centroid -0.1129).
    # Reconstruction: cos = C7 / sqrt(C7^2 + 127 C4^2) and relative L2 error
    # sqrt((1 - C7)^2 + 127 C4^2), whatever the constant.
    c7, c4 = 0.9816, 0.1129
    cos_cf = c7 / math.sqrt(c7 ** 2 + 127 * c4 ** 2)
    rel_cf = math.sqrt((1 - c7) ** 2 + 127 * c4 ** 2)
    assert round(cos_cf, 3) == 0.611 and round(rel_cf, 2) == 1.27
    for const in (2.5, -0.7, 3.0, 1e-3):
        x = np.full((4, 128), const, dtype=np.float32)
        xr = _round_trip(oracle_mod, x, signs, post_flip=True)
        cos = cosine_rows(x, xr).mean()
        rel = np.linalg.norm(xr - x) / np.linalg.norm(x)
        assert abs(cos - cos_cf) < 2e-4, cos
        assert abs(rel - rel_cf) < 2e-4, rel
        good = cosine_rows(x, _round_trip(oracle_mod, x, signs)).mean()
        assert good > 0.97


def test_post_flip_is_a_no_op_except_exact_ties(oracle_mod, signs):
    # A flip after the transform is undone exactly by the dequantiser, so the
    # reconstruction equals the one with no flips at all -- bit for bit --
    # unless a coefficient sits exactly on a boundary (then the tie goes to
    # the lower cell on both signs and the symmetry breaks).
    ones = np.ones(128, dtype=np.float32)
    x = datagen.gaussian_vectors(2048, seed=77).numpy()
    a = _round_trip(oracle_mod, x, signs, post_flip=True)
    b = _round_trip(oracle_mod, x, ones)
    _, bnd = oracle_mod.tq3_tables()
    xs = oracle_mod.tq3_scaled_coeffs(x, ones)
    tied = np.isin(xs, bnd).any(axis=1)
    assert np.array_equal(a[~tied], b[~tied])
    # constant blocks: every row carries exact zeros, and rows differ
    xc = np.full((8, 128), 1.5, dtype=np.float32)
    xsc = oracle_mod.tq3_scaled_coeffs(xc, ones)
    assert np.all((xsc == 0).sum(axis=1) == 127)
    assert not np.array_equal(_round_trip(oracle_mod, xc, signs, post_flip=True),
                              _round_trip(oracle_mod, xc, ones))


def test_norm_clamp_zero_vector(oracle_mod, signs):
    x = np.zeros((2, 128), dtype=np.float32)
    rec = oracle_mod.tq3_quantize(x, signs)
    _, norms, scales = oracle_mod.tq3_split(rec)
    assert np.all(norms == np.float32(1e-8)) and np.all(scales == np.float32(1e-8))
    assert np.all(oracle_mod.unpack(rec[0, :48], 128, 3) == 3)
