"""Pins of the oracle's FWHT against a brute-force dense Sylvester Hadamard.

Source: "ComfyUI-TurboQuant: tq3_core.py", _fwht_inplace (natural-order,
orthonormal, self-inverse transform) and its self-test [4]; "orbit_quant.py",
_fwht (the same transform on h-blocks).
"""
import numpy as np
import pytest


def sylvester(n):
    """Dense +-1 Hadamard in natural order: H_1 = [1], H_2m = [[H, H], [H, -H]]."""
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32, 64, 128, 1024])
def test_hadamard_orthogonal(n):
    h = sylvester(n)
    assert np.array_equal(h @ h, n * np.eye(n, dtype=np.int64))


@pytest.mark.parametrize("n", [8, 128, 1024])
def test_fwht_matches_dense(oracle_mod, n):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((16, n)).astype(np.float32)
    got = oracle_mod.fwht(x, "tq3" if n == 128 else "orbit")
    ref = (x.astype(np.float64) @ sylvester(n).T.astype(np.float64)) / np.sqrt(n)
    scale = np.linalg.norm(x.astype(np.float64), axis=1, keepdims=True)
    assert np.max(np.abs(got - ref) / scale) < 1e-6


def test_fwht_unit_vectors_give_columns(oracle_mod):
    # natural (Sylvester) ordering: FWHT(e_k) is column k of H/sqrt(128)
    e = np.eye(128, dtype=np.float32)
    got = oracle_mod.fwht(e)
    k = np.float32(1.0 / np.sqrt(128.0))
    assert np.array_equal(got, (sylvester(128).T * k).astype(np.float32))


def test_fwht_self_inverse(oracle_mod):
    # the TQ3 page's self-test [4]: max error below 1e-5 on randn(8, 128)
    rng = np.random.default_rng(123)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    back = oracle_mod.fwht(oracle_mod.fwht(x))
    assert np.max(np.abs(back - x)) < 1e-5


def test_orbit_normalisation_exact_power(oracle_mod):
    # h = 1024: h ** -0.5 = 2^-5 exactly, so FWHT(e_0) is exactly 1/32
    e = np.zeros((1, 1024), dtype=np.float32)
    e[0, 0] = 1.0
    assert np.all(oracle_mod.fwht(e, "orbit") == np.float32(1.0 / 32))
