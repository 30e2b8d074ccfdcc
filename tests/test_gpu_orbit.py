"""GPU parity of the OrbitQuant weight codec against the oracle.

Source: "zerogpu-sdxlTrainer: toolkit/util/orbit_quant.py" (_quantize_rows,
_dequantize_rotated, dequantize). Weights ~ N(0, 0.02^2); rotations from the
page's seed rule (datagen.rpbh_params). The library is handed its own codebook
(orbit_make_codebook) and the oracle its own (oracle.orbit_codebook); the two
are asserted equal for every (bits, d) used.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from parity_util import compare_reconstruction

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import randomized_hadamard_lloyd_amd as m
    return m


def edges_of(cb):
    c = np.asarray(cb, dtype=np.float32)
    return ((c[:-1] + c[1:]) / np.float32(2)).astype(np.float64)


def codebooks(tq, bits, d):
    """(library codebook, oracle codebook), asserted identical."""
    lib_cb = tq.orbit_make_codebook(bits, d)
    o_cb = oracle.orbit_codebook(bits, d)
    assert np.array_equal(lib_cb.numpy(), o_cb), (bits, d)
    return lib_cb, o_cb


def check(tq, w, d, bits, msb=True, dtype=torch.float32, full_check=True, cb=None):
    perm, sg = datagen.rpbh_params(d)
    inv = torch.argsort(perm)
    if cb is None:
        cb, o_cb = codebooks(tq, bits, d)
    else:
        o_cb = np.asarray(cb, dtype=np.float32)   # an explicit input, given to both sides
    order = tq.TQ_MSB_FIRST if msb else tq.TQ_LSB_FIRST
    packed, norms = tq.orbit_quantize_weight(w.to(DEV), bits, perm.to(DEV), sg.to(DEV), cb,
                                             bit_order=order)
    torch.cuda.synchronize()
    o_packed, o_norms = oracle.orbit_quantize(w.numpy(), bits, perm, sg, o_cb,
                                              msb_first=msb)
    g_norms = norms.cpu().numpy()
    assert np.max(np.abs(g_norms - o_norms) / np.maximum(o_norms, 1e-30)) <= 1e-6
    g_packed = packed.cpu().numpy()
    if not np.array_equal(g_packed, o_packed):
        rows = w.shape[0]
        gc = oracle.unpack(g_packed, rows * d, bits, msb_first=msb).reshape(rows, d)
        oc = oracle.unpack(o_packed, rows * d, bits, msb_first=msb).reshape(rows, d)
        unit, _ = oracle.orbit_unit(w.numpy(), perm, sg)
        diff = gc != oc
        dist = np.min(np.abs(unit[..., None].astype(np.float64) - edges_of(o_cb)), axis=-1)
        assert not (diff & (dist >= 1e-5 * np.abs(unit).max())).any(), "flips away from edges"
        assert diff.sum() <= 1e-6 * rows * d
        pytest.fail(f"codes not bit-identical: {int(diff.sum())} near-edge flips")
    assert np.array_equal(g_norms, o_norms)
    if not full_check:
        return packed, norms
    for rotated in (True, False):
        out = tq.orbit_dequantize(packed, norms, d, bits, inv.to(DEV), sg.to(DEV), cb,
                                  bit_order=order, rotated_only=rotated, dtype=dtype)
        torch.cuda.synchronize()
        ref = oracle.orbit_dequantize(o_packed, o_norms, d, bits, inv, sg, o_cb,
                                      msb_first=msb, rotated_only=rotated)
        st = compare_reconstruction(out, ref, o_norms, dtype)
        assert st["exact"], (rotated, st)
    return packed, norms


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("msb", [True, False])
def test_orbit_3072(tq, bits, msb):
    w = datagen.orbit_weight(rows=257, d=3072, seed=60 + bits)
    check(tq, w, 3072, bits, msb)


@pytest.mark.parametrize("d", [32, 96, 160, 256, 512, 768, 1024, 1536, 2048, 2560, 4096])
def test_orbit_dims(tq, d):
    # every Hadamard block size from 32 to 4096, partial and multi-tile rows
    w = datagen.orbit_weight(rows=67, d=d, seed=d)
    check(tq, w, d, 3)


@pytest.mark.parametrize("msb", [True, False])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [4608, 5120, 5632, 6144, 8192, 12288, 14336, 16384])
def test_orbit_large_d(tq, d, bits, msb):
    """Rows longer than 4096 ("orbit_quant.py", hadamard_block_size: the block
    is d & -d, here 512, 1024, 512, 2048, 8192, 4096, 2048 and 16384):
    blocks of up to 16 waves (5 and 6 waves with the sign masks rebuilt per
    row), Hadamard stages across waves up to index bit 13, tile sums of
    squares combined by the pairwise tree inside each block."""
    w = datagen.orbit_weight(rows=37, d=d, seed=d + bits)
    check(tq, w, d, bits, msb)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_orbit_large_d_narrow_outputs(tq, dtype):
    w = datagen.orbit_weight(rows=20, d=12288, seed=12)
    check(tq, w, 12288, 3, True, dtype)


def test_orbit_large_d_limits(tq):
    d = 16384 + 32                       # h = 32, one row longer than a block holds
    perm, sg = datagen.rpbh_params(d)
    cb = tq.orbit_make_codebook(3, d)
    with pytest.raises(ValueError):
        tq.orbit_quantize_weight(torch.zeros((2, d), device=DEV), 3, perm.to(DEV), sg.to(DEV), cb)
    with pytest.raises(ValueError):
        tq.orbit_rotate(torch.zeros((2, d), device=DEV), perm.to(DEV), sg.to(DEV))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_orbit_narrow_outputs(tq, dtype):
    w = datagen.orbit_weight(rows=64, d=3072, seed=7)
    check(tq, w, 3072, 4, True, dtype)


def test_orbit_edge_rows(tq):
    d = 3072
    w = datagen.orbit_weight(rows=8, d=d, seed=3)
    w[0] = 0.0                       # zero row: norm 0, every code from u = 0
    w[1] = 1.0                       # constant row
    w[2, ::7] = 0.0                  # exact zeros in a row
    w[3] = w[3] * 1e-20              # tiny row
    w[4] = w[4] * 1e15               # large row
    w[5, 100] = 50.0                 # outlier
    check(tq, w, d, 3)
    check(tq, w, d, 2, msb=False)


@pytest.mark.parametrize("d", [96, 1056, 3072, 4096, 12288])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("msb", [True, False])
def test_orbit_asymmetric_codebook(tq, d, bits, msb):
    """Codebooks that are not mirror-symmetric take the general edge count (the
    Gaussian ones take the symmetric compare), in kernels of their own for
    every wave count: a shifted Gaussian codebook and an uneven random
    ascending one. d = 96 and 1056 leave lanes past the row's end."""
    w = datagen.orbit_weight(rows=129 if d <= 4096 else 33, d=d, seed=20 + bits)
    base = torch.from_numpy(codebooks(tq, bits, d)[1])
    shifted = base + np.float32(0.37) * (base[1] - base[0])
    rng = np.random.default_rng(bits)
    rand = torch.from_numpy(np.sort(rng.normal(0.0, 1.5 / np.sqrt(d), 1 << bits))
                            .astype(np.float32))
    for cb in (shifted, rand):
        assert not all(cb[k] == -cb[len(cb) - 1 - k] for k in range(len(cb)))
        check(tq, w, d, bits, msb, cb=cb)


def test_orbit_exact_zero_coefficients(tq):
    """Rows whose permuted, sign-flipped values are constant: every block's
    transform is zero except its first coefficient, so most u are exactly 0
    (the middle edge of a symmetric codebook; a tie that goes down) and the
    division takes its plain IEEE path."""
    d = 3072
    perm, sg = datagen.rpbh_params(d)
    inv = torch.argsort(perm)
    c = torch.tensor([1.0, -2.0, 0.5, 3.0, -0.25, 1e-3])[:, None]
    w = (c * sg[inv].to(torch.float32)[None, :]).contiguous()
    for bits in (2, 3, 4):
        check(tq, w, d, bits, True)
        check(tq, w, d, bits, False)


def test_orbit_errors(tq):
    d = 3072
    w = torch.zeros((4, d), device=DEV)
    perm, sg = datagen.rpbh_params(d)
    cb = tq.orbit_make_codebook(3, d)
    with pytest.raises(ValueError):
        tq.orbit_quantize_weight(w, 5, perm.to(DEV), sg.to(DEV), cb)       # bits
    with pytest.raises(ValueError):
        tq.orbit_quantize_weight(torch.zeros((4, 48), device=DEV), 3,      # h = 16
                                 perm[:48].to(DEV), sg[:48].to(DEV), cb)
    packed, norms = tq.orbit_quantize_weight(torch.zeros((0, d), device=DEV), 3,
                                             perm.to(DEV), sg.to(DEV), cb)
    assert packed.shape == (0, d * 3 // 8) and norms.shape == (0,)


def test_orbit_full_weight(tq):
    """The 12288 x 3072 weight at 2, 3 and 4 bits; every code and norm checked,
    reconstructions checked on a sample of rows."""
    d = 3072
    w = datagen.orbit_weight()
    perm, sg = datagen.rpbh_params(d)
    inv = torch.argsort(perm)
    rows = torch.from_numpy(np.random.default_rng(5).choice(w.shape[0], 512, replace=False))
    for bits in (2, 3, 4):
        cb, o_cb = codebooks(tq, bits, d)
        packed, norms = tq.orbit_quantize_weight(w.to(DEV), bits, perm.to(DEV), sg.to(DEV), cb)
        full = tq.orbit_dequantize(packed, norms, d, bits, inv.to(DEV), sg.to(DEV), cb)
        torch.cuda.synchronize()
        o_packed, o_norms = oracle.orbit_quantize(w.numpy(), bits, perm, sg, o_cb)
        assert np.array_equal(norms.cpu().numpy(), o_norms), bits
        assert np.array_equal(packed.cpu().numpy(), o_packed), bits
        ref = oracle.orbit_dequantize(o_packed[rows.numpy()], o_norms[rows.numpy()], d, bits,
                                      inv, sg, o_cb)
        st = compare_reconstruction(full[rows.to(DEV)], ref, o_norms[rows.numpy()])
        assert st["exact"], (bits, st)


def test_orbit_requantize_in_place(tq):
    """requantize_ ("orbit_quant.py", OrbitQuantizer.requantize_): a new fp32
    weight goes through the layer's stored permutation, signs and codebook into
    its existing packed / row-norm buffers; the result is the oracle's
    quantization of the new weight, and the buffers keep their identity."""
    d, bits, rows = 768, 3, 96
    perm, sg = datagen.rpbh_params(d)
    cb, o_cb = codebooks(tq, bits, d)
    rng = np.random.default_rng(21)
    w1 = torch.from_numpy((rng.standard_normal((rows, d)) * 0.02).astype(np.float32))
    w2 = torch.from_numpy((rng.standard_normal((rows, d)) * 0.05).astype(np.float32))
    p_dev, s_dev = perm.to(DEV), sg.to(DEV)
    packed, norms = tq.orbit_quantize_weight(w1.to(DEV), bits, p_dev, s_dev, cb)
    ptrs = (packed.data_ptr(), norms.data_ptr())
    p2, n2 = tq.orbit_quantize_weight(w2.to(DEV), bits, p_dev, s_dev, cb,
                                      packed=packed, row_norms=norms)
    torch.cuda.synchronize()
    assert (p2.data_ptr(), n2.data_ptr()) == ptrs
    o_packed, o_norms = oracle.orbit_quantize(w2.numpy(), bits, perm, sg, o_cb)
    assert np.array_equal(packed.cpu().numpy(), o_packed)
    assert np.array_equal(norms.cpu().numpy(), o_norms)


def test_orbit_requantize_rejects_wrong_buffers(tq):
    d, bits, rows = 256, 2, 8
    perm, sg = datagen.rpbh_params(d)
    cb = tq.orbit_make_codebook(bits, d)
    w = torch.zeros((rows, d), device=DEV)
    small = torch.empty((rows, d * bits // 8 - 1), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        tq.orbit_quantize_weight(w, bits, perm.to(DEV), sg.to(DEV), cb, packed=small)
    with pytest.raises(ValueError):
        tq.orbit_quantize_weight(w, bits, perm.to(DEV), sg.to(DEV), cb,
                                 row_norms=torch.empty(rows, dtype=torch.float16, device=DEV))
