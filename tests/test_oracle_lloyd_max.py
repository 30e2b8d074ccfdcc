"""Pins of the oracle's Gaussian Lloyd-Max codebooks.

Source: "orbit_quant.py", gaussian_lloyd_max (quantile-midpoint start, a fixed
200 iterations of the midpoint/conditional-mean updates in fp64, then fp32).

Independent references:
  * J. Max, "Quantizing for minimum distortion", IRE Trans. Inf. Theory, 1960:
    optimal output levels and mean-squared errors of the Gaussian quantiser
    (the textbook table, to its printed precision);
  * the two Lloyd-Max conditions checked with numerical quadrature, which shares
    nothing with the closed-form update the procedure uses;
  * the page's fixed iteration count pinned by a second Lloyd iteration that
    forms each conditional mean by adaptive quadrature (scipy.integrate.quad)
    and starts from scipy's normal quantile function -- no closed-form
    density ratio, no erf, no NormalDist -- and by the 4-bit codebook the
    page's procedure yields after exactly 200 iterations, to six decimals.
"""
import math

import numpy as np
import pytest
from scipy import integrate, stats

# Max (1960), Gaussian, positive output levels and distortion (unit variance)
MAX_LEVELS = {
    2: [0.4528, 1.510],
    3: [0.2451, 0.7560, 1.344, 2.152],
    4: [0.1284, 0.3881, 0.6568, 0.9424, 1.256, 1.618, 2.069, 2.733],
}
MAX_MSE = {2: 0.1175, 3: 0.03454, 4: 0.009497}


def _pdf(t):
    return math.exp(-t * t / 2) / math.sqrt(2 * math.pi)


@pytest.mark.parametrize("bits", [2, 3])
def test_page_procedure_matches_max_table(oracle_mod, bits):
    c = oracle_mod.gaussian_lloyd_max(bits)
    pos = c[len(c) // 2:]
    for got, want in zip(pos, MAX_LEVELS[bits]):
        assert abs(got - want) <= 0.6 * 10 ** -(len(str(want).split(".")[1]))


def test_four_bit_converges_to_max_table(oracle_mod):
    # 200 iterations leave the 16-level codebook short of convergence; run
    # the same procedure to convergence and compare with the table.
    c = np.asarray(oracle_mod.gaussian_lloyd_max_f64(4, iters=20000))
    for got, want in zip(c[8:], MAX_LEVELS[4]):
        assert abs(got - want) < 0.6e-3
    c200 = oracle_mod.gaussian_lloyd_max(4)
    assert 1e-5 < np.max(np.abs(c200 - c)) < 1e-3   # the page's value differs


# The page's procedure evaluated with torch in fp64 (erfinv start, torch.erf /
# torch.exp updates, 200 iterations): the positive half of the 4-bit codebook,
# rounded to six decimals. 199 or 201 iterations move it by about 1.9e-5.
PAGE_4BIT_200 = [0.128324, 0.387841, 0.656431, 0.941915,
                 1.255739, 1.617524, 2.068505, 2.732137]


def _quadrature_lloyd(bits, iters):
    """Lloyd's iteration with every centroid formed as the quadrature of
    t * pdf over its cell divided by the quadrature of pdf."""
    levels = 2 ** bits
    c = [float(stats.norm.ppf((k + 0.5) / levels)) for k in range(levels)]
    for _ in range(iters):
        e = [-np.inf] + [(c[k] + c[k + 1]) / 2 for k in range(levels - 1)] + [np.inf]
        nxt = []
        for k in range(levels):
            mass = integrate.quad(_pdf, e[k], e[k + 1], epsabs=1e-15, epsrel=1e-13)[0]
            first = integrate.quad(lambda t: t * _pdf(t), e[k], e[k + 1],
                                   epsabs=1e-15, epsrel=1e-13)[0]
            nxt.append(first / mass)
        c = nxt
    return np.asarray(c)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_iteration_count_pinned_by_quadrature(oracle_mod, bits):
    ref = _quadrature_lloyd(bits, 200)
    got = np.asarray(oracle_mod.gaussian_lloyd_max_f64(bits, 200))
    assert np.max(np.abs(got - ref)) < 1e-11
    # the fp32 codebook is the rounding of that fp64 result
    assert np.array_equal(oracle_mod.gaussian_lloyd_max(bits), ref.astype(np.float32))
    if bits == 4:
        # the pin separates the page's 200 iterations from 199 and 201
        for n in (199, 201):
            other = np.asarray(oracle_mod.gaussian_lloyd_max_f64(bits, n))
            assert np.max(np.abs(other - ref)) > 1e-6, n


def _six_decimals_match(c):
    pos = np.asarray(c, dtype=np.float64)[8:]
    return bool(np.all(np.abs(pos - np.asarray(PAGE_4BIT_200)) <= 0.5e-6 + 1e-7))


def test_four_bit_200_iterations_to_six_decimals(oracle_mod):
    c = oracle_mod.gaussian_lloyd_max(4)
    assert _six_decimals_match(c)
    assert np.array_equal(c[:8], -c[8:][::-1])        # mirror-symmetric in fp32
    for n in (199, 201):
        assert not _six_decimals_match(oracle_mod.gaussian_lloyd_max(4, n)), n


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_lloyd_conditions_by_quadrature(oracle_mod, bits):
    c = np.asarray(oracle_mod.gaussian_lloyd_max_f64(bits, iters=20000))
    edges = np.concatenate([[-np.inf], (c[:-1] + c[1:]) / 2, [np.inf]])
    mse = 0.0
    for k in range(len(c)):
        lo, hi = edges[k], edges[k + 1]
        mass = integrate.quad(_pdf, lo, hi, epsabs=1e-14)[0]
        first = integrate.quad(lambda t: t * _pdf(t), lo, hi, epsabs=1e-14)[0]
        assert abs(first / mass - c[k]) < 1e-9
        mse += integrate.quad(lambda t: (t - c[k]) ** 2 * _pdf(t), lo, hi,
                              epsabs=1e-14)[0]
    assert abs(mse - MAX_MSE[bits]) < 0.6 * 10 ** -(len(str(MAX_MSE[bits]).split(".")[1]) - 1)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_codebook_is_ascending_and_scaled(oracle_mod, bits):
    c = oracle_mod.gaussian_lloyd_max(bits)
    assert c.dtype == np.float32 and c.size == 2 ** bits
    assert np.all(np.diff(c) > 0)
    cb = oracle_mod.orbit_codebook(bits, 3072)
    assert np.array_equal(cb, (c * np.float32(3072 ** -0.5)).astype(np.float32))
    e = oracle_mod.orbit_edges(cb)
    assert np.all((e > cb[:-1]) & (e < cb[1:]))


def test_tq3_table_is_not_a_scaled_gaussian_codebook(oracle_mod):
    # Reading: the printed 8-level TQ3 table is a format constant. No
    # rescaling of the 3-bit Gaussian codebook reproduces it to 4 decimals,
    # so the oracle enters it as printed.
    g = np.asarray(oracle_mod.gaussian_lloyd_max_f64(3))[4:]
    c, _ = oracle_mod.tq3_tables()
    ratio = c[4:] / g
    assert np.ptp(ratio) > 1e-3
