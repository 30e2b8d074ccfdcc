"""The library enqueues on the caller's stream and nowhere else.

Each entry point takes a hipStream_t; the Python binding passes torch's current
stream. On a side stream the results must match the oracle's, work must be
ordered after what that stream already holds, and the library must not
synchronize the device: launching behind a long spin kernel on the side
stream returns at once, while another stream stays free.
"""
import time

import numpy as np
import pytest
import torch

import datagen
import oracle
from oracle import attention as oatt

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import randomized_hadamard_lloyd_amd as m
    return m


def test_side_stream_results_and_ordering(tq):
    signs = datagen.tq3_signs()
    x = datagen.gaussian_vectors(5000, seed=21).to(DEV)
    side = torch.cuda.Stream(device=DEV)
    tq.tq3_dequantize(tq.tq3_quantize(x[:64], signs), signs)  # first launches load the code
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        torch.cuda._sleep(20_000_000)  # keeps the side stream busy for milliseconds
        t0 = time.perf_counter()
        rec = tq.tq3_quantize(x, signs)
        y = tq.tq3_dequantize(rec, signs)
        host_s = time.perf_counter() - t0
        done = torch.cuda.Event()
        done.record(side)
    # the calls only enqueued: they returned while the spin kernel still ran
    assert not done.query()
    assert host_s < 0.5
    side.synchronize()
    o = oracle.tq3_quantize(x.cpu().numpy(), signs)
    assert np.array_equal(rec.cpu().numpy().reshape(-1, 56), o)
    assert np.array_equal(y.cpu().numpy(), oracle.tq3_dequantize(o, signs))


def test_orbit_and_attention_on_side_stream(tq):
    d, bits = 768, 3
    perm, sg = datagen.rpbh_params(d)
    cb = tq.orbit_make_codebook(bits, d)
    o_cb = oracle.orbit_codebook(bits, d)
    assert np.array_equal(cb.numpy(), o_cb)
    w = (torch.randn(64, d, generator=torch.Generator().manual_seed(3)) * 0.02)
    signs = datagen.tq3_signs()
    hkv, group, n_tok = 2, 4, 300
    rng = np.random.default_rng(17)
    k_rec = oracle.tq3_quantize(rng.standard_normal((n_tok * hkv, 128)).astype(np.float32),
                                signs.numpy())
    v_rec = oracle.tq3_quantize(rng.standard_normal((n_tok * hkv, 128)).astype(np.float32),
                                signs.numpy())
    q = rng.standard_normal((hkv * group, 128)).astype(np.float32)
    side = torch.cuda.Stream(device=DEV)
    with torch.cuda.stream(side):
        wd = w.to(DEV, non_blocking=False)
        packed, norms = tq.orbit_quantize_weight(wd, bits, perm.to(DEV), sg.to(DEV), cb)
        xr = tq.orbit_rotate(torch.ones(4, d, device=DEV), perm.to(DEV), sg.to(DEV))
        att = tq.tq3_decode_attention(torch.from_numpy(q).to(DEV), torch.from_numpy(k_rec).to(DEV),
                                      torch.from_numpy(v_rec).to(DEV), hkv, signs)
    side.synchronize()
    o_packed, o_norms = oracle.orbit_quantize(w.numpy(), bits, perm, sg, o_cb)
    assert np.array_equal(packed.cpu().numpy(), o_packed)
    assert np.array_equal(norms.cpu().numpy(), o_norms)
    assert np.array_equal(xr.cpu().numpy(),
                          oracle.rpbh_forward(np.ones((4, d), np.float32), perm, sg))
    ref = oatt.tq3_decode_attention(q, k_rec, v_rec, hkv, signs.numpy(), 128 ** -0.5)
    vmax = np.abs(oatt.dequantized_cache(v_rec, hkv, signs.numpy())).max()
    # fp32 rounding of scores and sums, far inside the attention tests' bound
    assert np.abs(att.cpu().numpy().astype(np.float64) - ref).max() <= 1e-4 * vmax
