"""Gaussian Lloyd-Max codebook, the oracle's version (pure Python, fp64).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the benchmark's
CPU-baseline leg, never by the product package.

Follows the procedure of gaussian_lloyd_max on the page "zerogpu-sdxlTrainer:
toolkit/util/orbit_quant.py" (OrbitQuant backend), in its order:

  * L = 2**bits levels, initialised at the standard-normal quantiles of the
    cell midpoints q_k = (k + 1/2) / L (the page writes this as
    sqrt(2) * erfinv(2q - 1); here the same value comes from the inverse CDF);
  * a fixed number of iterations (200 by default, no early stop), each
    setting the edges to the midpoints of neighbouring centroids and every
    centroid to the mean of the standard normal restricted to its cell,
    (phi(lo) - phi(hi)) / (Phi(hi) - Phi(lo));
  * the result rounded to float32 after the loop.

Reading: the page's indentation is lost in extraction; the plain reading (the
edge, density, CDF and update lines form the loop body, the float32 cast follows
the loop) is the one used here.
"""
import math
from statistics import NormalDist

import numpy as np

_SQRT2 = math.sqrt(2.0)
_SQRT2PI = math.sqrt(2.0 * math.pi)


def _phi(t: float) -> float:
    # standard normal density; exp(-inf) = 0 at the open ends
    if math.isinf(t):
        return 0.0
    return math.exp(-t * t / 2.0) / _SQRT2PI


def _cdf(t: float) -> float:
    return 0.5 * (1.0 + math.erf(t / _SQRT2))


def gaussian_lloyd_max_f64(bits: int, iters: int = 200) -> list:
    """Centroids in fp64, ascending, after `iters` Lloyd iterations."""
    levels = 2 ** bits
    nd = NormalDist()
    c = [nd.inv_cdf((k + 0.5) / levels) for k in range(levels)]
    for _ in range(iters):
        edges = [(c[k] + c[k + 1]) / 2.0 for k in range(levels - 1)]
        lo = [-math.inf] + edges
        hi = edges + [math.inf]
        c = [(_phi(lo[k]) - _phi(hi[k])) / (_cdf(hi[k]) - _cdf(lo[k]))
             for k in range(levels)]
    return c


def gaussian_lloyd_max(bits: int, iters: int = 200) -> np.ndarray:
    """The page's codebook: fp64 iteration, then rounded to float32."""
    return np.asarray(gaussian_lloyd_max_f64(bits, iters), dtype=np.float32)


def orbit_codebook(bits: int, d: int) -> np.ndarray:
    """Codebook for the N(0, 1/d) coordinate marginal as OrbitQuantizer.quantize_
    forms it: the float32 standard-normal codebook times d ** -0.5, the scalar
    rounded to float32 and the product taken in float32."""
    scale = np.float32(d ** -0.5)
    return (gaussian_lloyd_max(bits) * scale).astype(np.float32)


def orbit_edges(codebook: np.ndarray) -> np.ndarray:
    """Decision edges of _quantize_rows: float32 midpoints of neighbours."""
    cb = np.asarray(codebook, dtype=np.float32)
    return ((cb[:-1] + cb[1:]) / np.float32(2.0)).astype(np.float32)
