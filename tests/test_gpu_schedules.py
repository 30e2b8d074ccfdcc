"""Schedule independence: every output row depends only on its own input row.

The kernels share state only inside a block (the OrbitQuant row staged in LDS,
block sums, wave-bit exchanges; the TQ3 centroid table), and the launchers size
their grids from the row or vector count, so the same row is processed by a
different block, at a different iteration of the grid-stride loop, next to
different neighbours, when the count changes. A missing barrier or a stale LDS
read would then show up as a row whose result depends on the launch. Each test
runs the same rows in several launches (prefixes, offsets, a permuted order,
counts on either side of the TQ3 pipelined-loop threshold, two streams at
once) and requires bit-identical results row by row. Correctness against the
oracle is covered elsewhere; this is the race check.
"""
import numpy as np
import pytest
import torch

import datagen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import randomized_hadamard_lloyd_amd as m
    return m


def row_subsets(rows, seed):
    rng = np.random.default_rng(seed)
    perm = torch.from_numpy(rng.permutation(rows))
    return [slice(0, 1), slice(0, 7), slice(3, rows // 3 + 3), slice(rows - 5, rows),
            slice(1, rows)], perm


@pytest.mark.parametrize("d", [96, 1056, 3072, 4096, 5120, 12288])
def test_orbit_codec_rows_independent(tq, d):
    rows = 777 if d <= 4096 else 201
    w = datagen.orbit_weight(rows=rows, d=d, seed=d).to(DEV)
    perm, sg = datagen.rpbh_params(d)
    perm_d, sg_d, inv_d = perm.to(DEV), sg.to(DEV), torch.argsort(perm).to(DEV)
    for bits in (2, 3):
        cb = tq.orbit_make_codebook(bits, d)
        pk, nr = tq.orbit_quantize_weight(w, bits, perm_d, sg_d, cb)
        full = tq.orbit_dequantize(pk, nr, d, bits, inv_d, sg_d, cb)
        rot = tq.orbit_dequantize(pk, nr, d, bits, inv_d, sg_d, cb, rotated_only=True)
        subsets, p = row_subsets(rows, d + bits)
        for sl in subsets + [p.to(DEV)]:
            pk2, nr2 = tq.orbit_quantize_weight(w[sl].contiguous(), bits, perm_d, sg_d, cb)
            assert torch.equal(pk2, pk[sl]) and torch.equal(nr2, nr[sl]), (d, bits, sl)
            assert torch.equal(tq.orbit_dequantize(pk2, nr2, d, bits, inv_d, sg_d, cb), full[sl])
            assert torch.equal(tq.orbit_dequantize(pk2, nr2, d, bits, inv_d, sg_d, cb,
                                                   rotated_only=True), rot[sl])


@pytest.mark.parametrize("d", [96, 1024, 3072, 8192])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_orbit_rotate_rows_independent(tq, d, dtype):
    rows = 531
    x = torch.randn(rows, d, generator=torch.Generator().manual_seed(d)).to(dtype).to(DEV)
    perm, sg = datagen.rpbh_params(d)
    perm_d, sg_d = perm.to(DEV), sg.to(DEV)
    ref = tq.orbit_rotate(x, perm_d, sg_d)
    subsets, p = row_subsets(rows, d)
    for sl in subsets + [p.to(DEV)]:
        assert torch.equal(tq.orbit_rotate(x[sl].contiguous(), perm_d, sg_d), ref[sl]), (d, sl)
    if dtype == torch.bfloat16:
        # the tiled form: whole row tiles of a prefix match the full run's
        full_t = tq.orbit_rotate_tiled(x, perm_d, sg_d)
        for k in (16, 48, 512):
            part = tq.orbit_rotate_tiled(x[:k].contiguous(), perm_d, sg_d)
            assert torch.equal(part, full_t[: k * d]), (d, k)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_tq3_vectors_independent(tq, dtype):
    """Counts on either side of the dequantizer's pipelined-loop threshold
    (about 2^20 vectors) and the quantizer's grid sizes."""
    signs = datagen.tq3_signs()
    n = (1 << 20) + 4099
    x = datagen.gaussian_vectors(n, seed=7).to(dtype).to(DEV)
    rec = tq.tq3_quantize(x, signs)
    y = tq.tq3_dequantize(rec, signs, dtype=dtype)
    for sl in (slice(0, 1), slice(5, 1000), slice(1 << 19, (1 << 19) + 65537),
               slice(n - (1 << 20), n), slice(1, n)):
        r2 = tq.tq3_quantize(x[sl].contiguous(), signs)
        assert torch.equal(r2, rec[sl]), sl
        assert torch.equal(tq.tq3_dequantize(r2, signs, dtype=dtype), y[sl]), sl


def test_two_streams_at_once(tq):
    """Two launches of each codec on separate streams, overlapping in time,
    give the serial results: no state shared between launches."""
    d, rows = 3072, 2048
    w = datagen.orbit_weight(rows=rows, d=d, seed=9).to(DEV)
    perm, sg = datagen.rpbh_params(d)
    perm_d, sg_d = perm.to(DEV), sg.to(DEV)
    cb = tq.orbit_make_codebook(3, d)
    signs = datagen.tq3_signs()
    x = datagen.gaussian_vectors(1 << 18, seed=8).to(torch.bfloat16).to(DEV)
    pk_ref, nr_ref = tq.orbit_quantize_weight(w, 3, perm_d, sg_d, cb)
    rec_ref = tq.tq3_quantize(x, signs)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            a = tq.orbit_quantize_weight(w, 3, perm_d, sg_d, cb)
            c = tq.tq3_quantize(x, signs)
        with torch.cuda.stream(s2):
            b = tq.orbit_quantize_weight(w, 3, perm_d, sg_d, cb)
            e = tq.tq3_quantize(x, signs)
        outs.append((a, b, c, e))
    torch.cuda.synchronize()
    for a, b, c, e in outs:
        for pk, nr in (a, b):
            assert torch.equal(pk, pk_ref) and torch.equal(nr, nr_ref)
        assert torch.equal(c, rec_ref) and torch.equal(e, rec_ref)
