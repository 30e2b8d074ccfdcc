"""Comparison helpers for GPU-vs-oracle parity tests.

Tolerances (the codec contract): norms and scales within 1e-6 relative;
packed indices bit-exact except where the oracle's scaled coefficient lies
within 1e-5 of a boundary -- such flips are counted and must stay below 1e-6
of all indices; reconstructions within 1e-5 x the vector (row) norm, max abs.
For bf16/fp16 outputs the reconstruction bound adds one ulp of the narrow
type at the oracle's value (the rounding of the narrowing itself).

The GPU path replicates the oracle's operation order, so every comparison
also reports whether the results are bit-identical; tests assert that too.
"""
import numpy as np
import torch

import oracle

TQ3_BOUNDS = oracle.tq3_tables()[1].astype(np.float64)


def unpack3(packed):
    """LSB-first 3-bit stream [n, 48] -> indices [n, 128] (np.unpackbits)."""
    bits = np.unpackbits(np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1, 48),
                         axis=1, bitorder="little")
    return (bits.reshape(-1, 128, 3).astype(np.int64) * np.array([1, 2, 4])).sum(-1)


def split_records(rec):
    rec = np.ascontiguousarray(rec, dtype=np.uint8).reshape(-1, 56)
    norms = rec[:, 48:52].copy().view(np.float32).reshape(-1)
    scales = rec[:, 52:56].copy().view(np.float32).reshape(-1)
    return rec[:, :48], norms, scales


def _rel_err(got, want):
    """Max relative error over finite reference values; non-finite reference
    values (a sum of squares that overflowed fp32) must be matched exactly."""
    got, want = np.asarray(got), np.asarray(want)
    fin = np.isfinite(want)
    assert np.array_equal(got[~fin], want[~fin]), "non-finite values differ"
    if not fin.any():
        return 0.0
    g, w = got[fin].astype(np.float64), want[fin].astype(np.float64)
    return float(np.max(np.abs(g - w) / np.abs(w)))


def compare_tq3_records(gpu_rec, orc_rec, scaled_coeffs):
    """Returns a dict of statistics and asserts the tolerance contract."""
    gp, gn, gs = split_records(gpu_rec)
    op, on, os_ = split_records(orc_rec)
    n_vec = on.size
    rel_n, rel_s = _rel_err(gn, on), _rel_err(gs, os_)
    gi, oi = unpack3(gp), unpack3(op)
    diff = gi != oi
    flips = int(diff.sum())
    if flips:
        xs = np.asarray(scaled_coeffs, dtype=np.float64).reshape(-1, 128)
        dist = np.min(np.abs(xs[..., None] - TQ3_BOUNDS), axis=-1)
        far = diff & (dist >= 1e-5)
        assert not far.any(), f"{int(far.sum())} index flips away from any boundary"
    total = n_vec * 128
    assert rel_n <= 1e-6, f"norm rel err {rel_n}"
    assert rel_s <= 1e-6, f"scale rel err {rel_s}"
    assert flips <= 1e-6 * total, f"{flips} near-boundary flips of {total} indices"
    return {"n": n_vec, "flips": flips, "norm_rel": float(rel_n), "scale_rel": float(rel_s),
            "exact": bool(np.array_equal(np.asarray(gpu_rec).reshape(-1, 56),
                                         np.asarray(orc_rec).reshape(-1, 56)))}


def narrow_ulp(ref_f32, dtype):
    """One ulp of `dtype` at each reference value's magnitude (0 for fp32).
    A correctly rounded narrow result is within half of it of the fp32 value."""
    if dtype == torch.float32:
        return np.zeros(np.shape(ref_f32), dtype=np.float64)
    t = torch.from_numpy(np.abs(np.ascontiguousarray(ref_f32, dtype=np.float32))).to(dtype)
    up = torch.nextafter(t, torch.full_like(t, float("inf")))
    return (up.to(torch.float64) - t.to(torch.float64)).numpy()


def compare_reconstruction(gpu_out, orc_f32, norms, dtype=torch.float32):
    """gpu_out: tensor/array [n, m]; orc_f32: oracle fp32 [n, m]; norms [n]."""
    g = gpu_out.to(torch.float64).cpu().numpy() if isinstance(gpu_out, torch.Tensor) \
        else np.asarray(gpu_out, dtype=np.float64)
    o = np.asarray(orc_f32, dtype=np.float64)
    nrm = np.asarray(norms, dtype=np.float64)
    fin = np.isfinite(nrm)
    if not fin.all():        # overflowed norms: values must match exactly
        assert np.array_equal(g[~fin], o[~fin], equal_nan=True)
        g, o, nrm, orc_f32 = g[fin], o[fin], nrm[fin], np.asarray(orc_f32)[fin]
        if isinstance(gpu_out, torch.Tensor):
            gpu_out = gpu_out[torch.from_numpy(fin).to(gpu_out.device)]
        norms = nrm
    err = np.abs(g - o)
    bound = 1e-5 * nrm[:, None] + narrow_ulp(orc_f32, dtype)
    assert np.all(err <= bound), f"max excess {np.max(err - bound)}"
    if dtype == torch.float32:
        exact = bool(np.array_equal(g, o))
    else:
        ref = torch.from_numpy(np.ascontiguousarray(orc_f32, dtype=np.float32)).to(dtype)
        exact = bool(torch.equal(gpu_out.cpu(), ref))
    scale = np.maximum(np.asarray(norms, dtype=np.float64), np.finfo(np.float64).tiny)
    return {"max_abs_over_norm": float(np.max(err / scale[:, None])) if err.size else 0.0,
            "exact": exact}
