"""GPU parity of the TQ3 codec on the three-array layout (tq3_quantize_split /
tq3_dequantize_split) and the page's dict form, against the oracle.

Source: "ComfyUI-TurboQuant: tq3_core.py": tq3_quantize returns a dict of
norms [..., D/128] fp32, scales [..., D/128] fp32, packed [..., D/128, 48]
uint8 and orig_shape; tq3_dequantize takes that dict back, checks its keys
and shapes, and returns fp32 in orig_shape. The oracle's records, split into
those three fields, are the expected values.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from parity_util import compare_reconstruction, compare_tq3_records

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import randomized_hadamard_lloyd_amd as m
    return m


@pytest.fixture(scope="module")
def signs():
    return datagen.tq3_signs()


def join(packed, norms, scales):
    """Three arrays -> [n, 56] records (the record layout of the oracle)."""
    p = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1, 48)
    n = np.ascontiguousarray(norms, dtype=np.float32).reshape(-1, 1).view(np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.float32).reshape(-1, 1).view(np.uint8)
    return np.concatenate([p, n, s], axis=1)


@pytest.mark.parametrize("n", [1, 3, 17, 64, 65, 1000, 4097])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_quantize_split_matches_oracle(tq, signs, n, dtype):
    x = datagen.gaussian_vectors(n, seed=300 + n).to(dtype)
    packed, norms, scales = tq.tq3_quantize_split(x.to(DEV), signs)
    torch.cuda.synchronize()
    assert packed.shape == (n, 1, 48) and norms.shape == (n, 1) and scales.shape == (n, 1)
    x32 = x.to(torch.float32).reshape(-1, 128).numpy()
    o = oracle.tq3_quantize(x32, signs)
    g = join(packed.cpu().numpy(), norms.cpu().numpy(), scales.cpu().numpy())
    st = compare_tq3_records(g, o, oracle.tq3_scaled_coeffs(x32, signs))
    assert st["exact"], st


@pytest.mark.parametrize("n", [1, 15, 16, 17, 63, 64, 65, 1000, 4097])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_dequantize_split_matches_oracle(tq, signs, n, dtype):
    x = datagen.gaussian_vectors(n, seed=400 + n).numpy()
    o = oracle.tq3_quantize(x, signs)
    op, on, os_ = oracle.tq3_split(o)
    y = tq.tq3_dequantize_split(torch.from_numpy(np.ascontiguousarray(op)).to(DEV),
                                torch.from_numpy(on).to(DEV), torch.from_numpy(os_).to(DEV),
                                signs, dtype=dtype)
    torch.cuda.synchronize()
    assert y.shape == (n * 128,)
    st = compare_reconstruction(y.reshape(-1, 128), oracle.tq3_dequantize(o, signs), on, dtype)
    assert st["exact"], st


def test_dict_round_trip_shapes(tq, signs):
    """[2, 3, 5, 384] -> dict with the page's shapes -> fp32 of orig_shape."""
    x = datagen.gaussian_vectors(2 * 3 * 5 * 3, seed=11).reshape(2, 3, 5, 384)
    d = tq.tq3_quantize_dict(x.to(DEV), signs)
    assert set(d) == {"norms", "scales", "packed", "orig_shape"}
    assert d["norms"].shape == (2, 3, 5, 3) and d["scales"].shape == (2, 3, 5, 3)
    assert d["packed"].shape == (2, 3, 5, 3, 48) and d["packed"].dtype == torch.uint8
    assert tuple(d["orig_shape"]) == (2, 3, 5, 384)
    o = oracle.tq3_quantize(x.reshape(-1, 128).numpy(), signs)
    op, on, os_ = oracle.tq3_split(o)
    assert np.array_equal(d["packed"].cpu().numpy().reshape(-1, 48), op)
    assert np.array_equal(d["norms"].cpu().numpy().reshape(-1), on)
    assert np.array_equal(d["scales"].cpu().numpy().reshape(-1), os_)
    y = tq.tq3_dequantize_dict(d, signs)
    assert y.shape == (2, 3, 5, 384) and y.dtype == torch.float32
    assert np.array_equal(y.cpu().numpy().reshape(-1, 128), oracle.tq3_dequantize(o, signs))


def test_dict_errors_as_on_the_page(tq, signs):
    d = tq.tq3_quantize_dict(datagen.gaussian_vectors(8, seed=1).to(DEV), signs)
    with pytest.raises(KeyError):
        tq.tq3_dequantize_dict({k: v for k, v in d.items() if k != "scales"}, signs)
    bad = dict(d, scales=d["scales"][:4])
    with pytest.raises(ValueError):
        tq.tq3_dequantize_dict(bad, signs)
    bad = dict(d, packed=d["packed"][..., :40])
    with pytest.raises(ValueError):
        tq.tq3_dequantize_dict(bad, signs)
    with pytest.raises(TypeError):
        tq.tq3_dequantize_dict(dict(d, norms=d["norms"].half()), signs)
    z = torch.zeros((0, 128), device=DEV)
    p, n, s = tq.tq3_quantize_split(z, signs)
    assert p.shape == (0, 1, 48) and n.shape == (0, 1)
    assert tq.tq3_dequantize_split(p, n, s, signs).shape == (0, 128)
    L, m = tq.lib, tq.sign_mask(signs)
    x = torch.zeros((4, 128), device=DEV)
    pk = torch.empty((4, 48), dtype=torch.uint8, device=DEV)
    nr = torch.empty(5, device=DEV)
    assert L.tq3_quantize_split(tq._ptr(x), 0, 4, 128, m, tq._ptr(pk), None, None, None) == 1
    assert L.tq3_quantize_split(tq._ptr(x), 0, 4, 128, m, tq._ptr(pk), nr.data_ptr() + 2,
                                tq._ptr(nr), None) == 6


def test_full_kv_layer_split(tq, signs):
    """The K half of one layer (262144 bf16 vectors, [32768, 8, 128]) through
    the three-array layout: every field of every vector, then a sample back."""
    x = datagen.kv_cache("K")
    packed, norms, scales = tq.tq3_quantize_split(x.to(DEV), signs)
    torch.cuda.synchronize()
    x32 = x.to(torch.float32).reshape(-1, 128).numpy()
    o = oracle.tq3_quantize(x32, signs)
    g = join(packed.cpu().numpy(), norms.cpu().numpy(), scales.cpu().numpy())
    if not np.array_equal(g, o):
        pytest.fail(f"not bit-identical: {compare_tq3_records(g, o, oracle.tq3_scaled_coeffs(x32, signs))}")
    y = tq.tq3_dequantize_split(packed, norms, scales, signs, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    y = y.reshape(-1, 128)
    idx = np.random.default_rng(3).choice(o.shape[0], 8192, replace=False)
    _, on, _ = oracle.tq3_split(o[idx])
    st = compare_reconstruction(y[torch.from_numpy(idx).to(DEV)], oracle.tq3_dequantize(o[idx], signs),
                                on, torch.bfloat16)
    assert st["exact"], st
