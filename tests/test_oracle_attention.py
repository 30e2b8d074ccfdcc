"""Pins of the decode-attention oracle against closed forms and invariants.

Source: "ComfyUI-TurboQuant: tq3_core.py" (TQ3 as a KV-cache codec: attention
reads the vectors tq3_dequantize reconstructs). Each pin fixes the oracle's
attention step by a case whose answer does not depend on its softmax code:
a single token, a zero softmax scale, duplicated keys, a dominant key, token
order, and the grouping of query heads onto KV heads.
"""
import numpy as np
import pytest

import datagen
import oracle
from oracle import attention as oatt

SIGNS = datagen.tq3_signs().numpy()


def records(n, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 128)).astype(np.float32) * np.float32(scale)
    return oracle.tq3_quantize(x, SIGNS)


def queries(hq, seed):
    return np.random.default_rng(seed).standard_normal((hq, 128)).astype(np.float32)


def test_single_token_returns_its_value():
    hkv, hq = 2, 8
    k, v = records(hkv, 1), records(hkv, 2)
    out = oatt.tq3_decode_attention(queries(hq, 3), k, v, hkv, SIGNS, 0.0883883)
    vd = oracle.tq3_dequantize(v, SIGNS).reshape(1, hkv, 128)
    for h in range(hq):
        assert np.array_equal(out[h], vd[0, h // (hq // hkv)].astype(np.float64))


def test_zero_scale_is_the_mean_value():
    hkv, hq, t = 2, 4, 37
    k, v = records(t * hkv, 4), records(t * hkv, 5)
    out = oatt.tq3_decode_attention(queries(hq, 6), k, v, hkv, SIGNS, 0.0)
    vd = oracle.tq3_dequantize(v, SIGNS).astype(np.float64).reshape(t, hkv, 128)
    for h in range(hq):
        assert np.allclose(out[h], vd[:, h // 2, :].mean(axis=0), rtol=0, atol=1e-12)


def test_duplicate_keys_share_weight_equally():
    k1 = records(1, 7)
    k = np.concatenate([k1, k1])  # T = 2, one KV head, identical keys
    v = records(2, 8)
    out = oatt.tq3_decode_attention(queries(1, 9), k, v, 1, SIGNS, 0.5)
    vd = oracle.tq3_dequantize(v, SIGNS).astype(np.float64)
    assert np.allclose(out[0], 0.5 * (vd[0] + vd[1]), rtol=0, atol=1e-12)


def test_dominant_key_selects_its_value():
    q = queries(1, 10)
    t = 50
    rng = np.random.default_rng(11)
    keys = rng.standard_normal((t, 128)).astype(np.float32) * 0.01
    keys[17] = q[0] * 50.0  # score about 50 * |q|^2 above the rest
    k = oracle.tq3_quantize(keys, SIGNS)
    v = records(t, 12)
    out = oatt.tq3_decode_attention(q, k, v, 1, SIGNS, 1.0)
    vd = oracle.tq3_dequantize(v, SIGNS).astype(np.float64)
    assert np.allclose(out[0], vd[17], rtol=0, atol=1e-12)


def test_token_order_does_not_matter():
    hkv, hq, t = 2, 4, 29
    k, v = records(t * hkv, 13), records(t * hkv, 14)
    q = queries(hq, 15)
    out = oatt.tq3_decode_attention(q, k, v, hkv, SIGNS, 0.09)
    perm = np.random.default_rng(16).permutation(t)
    kp = k.reshape(t, hkv, 56)[perm].reshape(-1, 56)
    vp = v.reshape(t, hkv, 56)[perm].reshape(-1, 56)
    outp = oatt.tq3_decode_attention(q, kp, vp, hkv, SIGNS, 0.09)
    assert np.allclose(out, outp, rtol=1e-12, atol=1e-14)


def test_query_heads_group_onto_kv_heads():
    hkv, group, t = 3, 4, 21
    k, v = records(t * hkv, 17), records(t * hkv, 18)
    q = queries(hkv * group, 19)
    out = oatt.tq3_decode_attention(q, k, v, hkv, SIGNS, 0.1)
    kr, vr = k.reshape(t, hkv, 56), v.reshape(t, hkv, 56)
    for h in range(hkv * group):
        j = h // group
        single = oatt.tq3_decode_attention(q[h:h + 1], kr[:, j], vr[:, j], 1, SIGNS, 0.1)
        assert np.array_equal(out[h], single[0])


def test_rejects_bad_shapes():
    k = records(6, 20)
    with pytest.raises(ValueError):
        oatt.tq3_decode_attention(queries(3, 21), k, k, 2, SIGNS, 0.1)  # 3 % 2 != 0
    with pytest.raises(ValueError):
        oatt.tq3_decode_attention(queries(2, 22), k, k[:4], 2, SIGNS, 0.1)
