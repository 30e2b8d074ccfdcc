"""The allocation-free attention entry point, tq3_decode_attention_noalloc.

It is tq3_decode_attention with the per-chunk partial results in a
library-held per-GPU array instead of a caller workspace, for callers that
cannot allocate. Both entry points run the same kernels, so the results must
be identical bit for bit; they are also held to the attention tests' bound
against the oracle (fp64 softmax attention over the oracle's reconstructions,
"ComfyUI-TurboQuant: tq3_core.py" tq3_dequantize). Two calls run back to back
on the shared array, each smaller than the one before.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
from oracle import attention as oatt

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
U = 2.0 ** -24


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import randomized_hadamard_lloyd_amd as m
    return m


def case(n_tok, hkv, group, seed, signs):
    rng = np.random.default_rng(seed)
    k = oracle.tq3_quantize(rng.standard_normal((n_tok * hkv, 128)).astype(np.float32), signs)
    v = oracle.tq3_quantize(rng.standard_normal((n_tok * hkv, 128)).astype(np.float32), signs)
    q = rng.standard_normal((hkv * group, 128)).astype(np.float32)
    return q, k, v


def noalloc_c_call(tq, q, k, v, hkv, mask, scale, out, odt):
    """Straight through the C ABI: plain device pointers, the current stream."""
    return tq.lib.tq3_decode_attention_noalloc(
        ctypes.c_void_p(q.data_ptr()), tq.TQ_F32 if q.dtype == torch.float32 else tq.TQ_BF16,
        q.shape[0], ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
        k.shape[0] // hkv, hkv, mask, ctypes.c_float(scale), ctypes.c_void_p(out.data_ptr()),
        odt, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def within_oracle_bound(got, q, k, v, hkv, signs, scale, odtype):
    ref = oatt.tq3_decode_attention(q, k, v, hkv, signs, scale)
    kd = oatt.dequantized_cache(k, hkv, signs).astype(np.float64)
    vd = oatt.dequantized_cache(v, hkv, signs).astype(np.float64)
    g = q.shape[0] // hkv
    for h in range(q.shape[0]):
        j = h // g
        a = abs(scale) * np.linalg.norm(q[h]) * np.linalg.norm(kd[:, j, :], axis=1).max()
        vmax = np.abs(vd[:, j, :]).max()
        tol = (1e-5 + 4 * math.sqrt(128) * U * a) * vmax
        if odtype != torch.float32:
            tol += np.abs(ref[h]).max() * 2.0 ** -8
        assert np.abs(got[h] - ref[h]).max() <= tol, h


@pytest.mark.parametrize("qdtype,odtype", [(torch.float32, torch.float32),
                                           (torch.bfloat16, torch.bfloat16)])
def test_noalloc_matches_workspace_entry_point(tq, qdtype, odtype):
    signs = datagen.tq3_signs().numpy()
    mask = tq.sign_mask(signs)
    scale = 128 ** -0.5
    odt = tq.TQ_F32 if odtype == torch.float32 else tq.TQ_BF16
    # three calls in a row on the shared array, each smaller than the one
    # before: 40000 tokens x 8 KV heads with 16 query heads (96 chunks of two
    # pieces), 8192 tokens x 8 KV heads with 32 (128 chunks of one piece),
    # then 1000 tokens x 2 KV heads with 8
    for n_tok, hkv, group, seed in ((40000, 8, 2, 3), (8192, 8, 4, 1), (1000, 2, 4, 2)):
        q, k, v = case(n_tok, hkv, group, seed, signs)
        need = tq.tq3_attention_workspace_bytes(n_tok, hkv * group, hkv)
        assert 0 < need <= tq.tq3_attention_noalloc_max_bytes()
        qd = torch.from_numpy(q).to(DEV, qdtype)
        kd, vd = torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV)
        ref = tq.tq3_decode_attention(qd, kd, vd, hkv, signs, scale, dtype=odtype)
        out = torch.full((hkv * group, 128), float("nan"), dtype=odtype, device=DEV)
        print(f"noalloc n_tok={n_tok} hkv={hkv} hq={hkv * group} {qdtype}", flush=True)
        st = noalloc_c_call(tq, qd, kd, vd, hkv, mask, scale, out, odt)
        assert st == 0, tq.lib.tq_status_str(st)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16 if odtype != torch.float32 else torch.int32),
                           ref.view(torch.int16 if odtype != torch.float32 else torch.int32))
        qq = qd.float().cpu().numpy()
        within_oracle_bound(out.float().cpu().numpy().astype(np.float64), qq, k, v, hkv, signs,
                            scale, odtype)


def test_noalloc_binding_and_size_limit(tq):
    signs = datagen.tq3_signs().numpy()
    q, k, v = case(300, 4, 2, 3, signs)
    qd = torch.from_numpy(q).to(DEV)
    kd, vd = torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV)
    a = tq.tq3_decode_attention_noalloc(qd, kd, vd, 4, signs)
    b = tq.tq3_decode_attention(qd, kd, vd, 4, signs)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # sizes whose partial results exceed the array are refused before any launch
    # (the buffers are never read): 32768 KV heads of one query head each, one
    # chunk per head, 32768 partials of 528 bytes
    n_tok, heads = 16, 32768
    assert tq.tq3_attention_workspace_bytes(n_tok, heads, heads) > tq.tq3_attention_noalloc_max_bytes()
    assert tq.tq3_attention_workspace_bytes(1 << 20, 32, 8) <= tq.tq3_attention_noalloc_max_bytes()
    out = torch.empty((32, 128), device=DEV)
    st = tq.lib.tq3_decode_attention_noalloc(
        ctypes.c_void_p(out.data_ptr()), tq.TQ_F32, heads, ctypes.c_void_p(kd.data_ptr()),
        ctypes.c_void_p(vd.data_ptr()), n_tok, heads, tq.sign_mask(signs), ctypes.c_float(0.1),
        ctypes.c_void_p(out.data_ptr()), tq.TQ_F32, None)
    assert st == 9
