"""Oracle for decode attention over a TQ3-compressed KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "ComfyUI-TurboQuant: tq3_core.py", module docstring: TQ3 compresses
the 128-float K and V vectors of a KV cache; attention then consumes the
reconstructed vectors that tq3_dequantize returns. The pages give no fused
kernel, so the oracle is the plain definition: every record is dequantized
exactly as tq3_dequantize does (the C oracle, fp32), and one decode step of
scaled dot-product attention is evaluated in fp64 on those vectors:

    s_t = softmax_scale * <q_h, K_t>,   p = softmax(s),   o_h = sum_t p_t V_t

for each query head h, reading KV head h // (Hq / Hkv) (grouped-query
attention: consecutive query heads share a KV head).

Cache layout: token-major, record (t * Hkv + j) holds token t of KV head j,
the layout of a [T, Hkv, 128] cache quantized row by row.
"""
import numpy as np

from . import tq3_dequantize


def tq3_decode_attention(q, k_records, v_records, n_kv_heads, signs, softmax_scale,
                         threads=0):
    """q: [Hq, 128]; k_records, v_records: uint8 [T * Hkv, 56]; signs: [128]
    of +-1. Returns fp64 [Hq, 128]."""
    q = np.asarray(q, dtype=np.float64).reshape(-1, 128)
    hq = q.shape[0]
    hkv = int(n_kv_heads)
    if hkv < 1 or hq % hkv != 0:
        raise ValueError("the query heads must split evenly over the KV heads")
    group = hq // hkv
    k = tq3_dequantize(k_records, signs, threads=threads).astype(np.float64)
    v = tq3_dequantize(v_records, signs, threads=threads).astype(np.float64)
    if k.shape[0] != v.shape[0] or k.shape[0] % hkv != 0 or k.shape[0] == 0:
        raise ValueError("K and V must hold the same nonzero number of tokens")
    t = k.shape[0] // hkv
    k = k.reshape(t, hkv, 128)
    v = v.reshape(t, hkv, 128)
    out = np.zeros((hq, 128), dtype=np.float64)
    for h in range(hq):
        j = h // group
        s = float(softmax_scale) * (k[:, j, :] @ q[h])
        s = s - s.max()
        p = np.exp(s)
        p = p / p.sum()
        out[h] = p @ v[:, j, :]
    return out


def dequantized_cache(records, n_kv_heads, signs, threads=0):
    """[T, Hkv, 128] fp32 vectors the attention reads (tq3_dequantize)."""
    y = tq3_dequantize(records, signs, threads=threads)
    return y.reshape(-1, int(n_kv_heads), 128)
