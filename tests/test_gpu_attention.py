"""GPU parity of decode attention over TQ3 records against the oracle.

The oracle (oracle/attention.py) dequantizes every record as
"ComfyUI-TurboQuant: tq3_core.py" tq3_dequantize does and evaluates
softmax attention in fp64. The kernels score and accumulate in the rotated
domain in fp32, so results agree to fp32 rounding: the bound used here is
  |o - o_ref| <= (1e-5 + 4 sqrt(128) u A) * max|V|,  u = 2^-24,
with A = |scale| * |q_h| * max_t |K_t| the largest possible score magnitude
of the head (the score error grows with it) and max|V| over the head's values.
"""
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


@pytest.fixture(scope="module")
def signs():
    return datagen.tq3_signs().numpy()


def run(tq, q, k_rec, v_rec, hkv, signs, scale, qdtype=torch.float32, odtype=torch.float32):
    """Kernel output (fp64) and the query it saw, rounded to qdtype."""
    out = tq.tq3_decode_attention(torch.from_numpy(q).to(DEV, qdtype),
                                  torch.from_numpy(k_rec).to(DEV), torch.from_numpy(v_rec).to(DEV),
                                  hkv, signs, scale, dtype=odtype)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    return got, torch.from_numpy(q).to(qdtype).float().numpy()


def check(tq, q, k_rec, v_rec, hkv, signs, scale, qdtype=torch.float32, odtype=torch.float32):
    got, qq = run(tq, q, k_rec, v_rec, hkv, signs, scale, qdtype, odtype)
    return compare(got, qq, k_rec, v_rec, hkv, signs, scale, odtype)


def compare(got, qq, k_rec, v_rec, hkv, signs, scale, odtype=torch.float32):
    hq = qq.shape[0]
    ref = oatt.tq3_decode_attention(qq, k_rec, v_rec, hkv, signs, scale)
    kd = oatt.dequantized_cache(k_rec, hkv, signs).astype(np.float64)
    vd = oatt.dequantized_cache(v_rec, hkv, signs).astype(np.float64)
    g = hq // hkv
    worst = 0.0
    for h in range(hq):
        j = h // g
        a = abs(scale) * np.linalg.norm(qq[h]) * np.linalg.norm(kd[:, j, :], axis=1).max()
        vmax = np.abs(vd[:, j, :]).max()
        tol = (1e-5 + 4 * math.sqrt(128) * U * a) * vmax
        if odtype != torch.float32:
            tol += np.abs(ref[h]).max() * (2.0 ** -8 if odtype == torch.bfloat16 else 2.0 ** -11)
        err = np.abs(got[h] - ref[h]).max()
        assert err <= tol, (h, err, tol, a)
        worst = max(worst, err / max(vmax, 1e-30))
    return worst


def gaussian_records(n, seed, signs, scale=1.0):
    x = np.random.default_rng(seed).standard_normal((n, 128)).astype(np.float32) * scale
    return oracle.tq3_quantize(x, signs)


@pytest.mark.parametrize("t", [1, 2, 15, 16, 17, 100, 1000, 4097])
@pytest.mark.parametrize("hkv,group", [(1, 1), (2, 4), (8, 4), (3, 8), (4, 2)])
def test_sizes_and_groups(tq, signs, t, hkv, group):
    hq = hkv * group
    q = np.random.default_rng(t * 7 + hkv).standard_normal((hq, 128)).astype(np.float32)
    k = gaussian_records(t * hkv, 100 + t, signs)
    v = gaussian_records(t * hkv, 200 + t, signs)
    check(tq, q, k, v, hkv, signs, 128 ** -0.5)


@pytest.mark.parametrize("qdtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("odtype", [torch.float32, torch.bfloat16, torch.float16])
def test_dtypes(tq, signs, qdtype, odtype):
    hkv, hq, t = 2, 8, 300
    q = np.random.default_rng(5).standard_normal((hq, 128)).astype(np.float32)
    check(tq, q, gaussian_records(t * hkv, 6, signs), gaussian_records(t * hkv, 7, signs), hkv,
          signs, 0.1, qdtype, odtype)


@pytest.mark.parametrize("hq", [32, 64])
def test_kv_layer_full_size(tq, signs, hq):
    """The KV-cache workload: K and V of one layer (32768 tokens x 8 KV heads,
    bf16 with outlier channels and per-token scales), quantized by the
    oracle, attended by 32 or 64 query heads (64: chunks of 512 tokens, two
    pieces each)."""
    k = oracle.tq3_quantize(datagen.kv_cache("K").float().numpy().reshape(-1, 128), signs)
    v = oracle.tq3_quantize(datagen.kv_cache("V").float().numpy().reshape(-1, 128), signs)
    q = datagen.attention_queries(hq).numpy()
    worst = check(tq, q, k, v, 8, signs, 128 ** -0.5)
    print(f"max |o - o_ref| / max|V| = {worst:.3e}")


@pytest.mark.parametrize("t,hkv", [(20000, 8), (40000, 4), (4500, 32)])
def test_eight_heads_long_chunks(tq, signs, t, hkv):
    """Eight query heads per KV head take chunks longer than 256 tokens,
    processed in pieces of 256: here 320-token chunks (a 64-token last piece)
    and a shorter last chunk, and 288-token chunks over 32 KV heads."""
    q = np.random.default_rng(t).standard_normal((8 * hkv, 128)).astype(np.float32)
    k = gaussian_records(t * hkv, 300 + hkv, signs)
    v = gaussian_records(t * hkv, 400 + hkv, signs)
    check(tq, q, k, v, hkv, signs, 128 ** -0.5)


@pytest.mark.parametrize("t,hkv,group", [(5000, 64, 4), (40000, 8, 2), (33000, 8, 1)])
def test_long_caches_in_pieces(tq, signs, t, hkv, group):
    """Up to 4 query heads per KV head, caches long enough that 1024 chunks
    would exceed 256 tokens take 768 chunks of several pieces: 432, 432 and
    352 tokens here (two pieces each, a short last piece and last chunk)."""
    q = np.random.default_rng(t + hkv).standard_normal((group * hkv, 128)).astype(np.float32)
    k = gaussian_records(t * hkv, 500 + hkv, signs)
    v = gaussian_records(t * hkv, 600 + hkv, signs)
    check(tq, q, k, v, hkv, signs, 128 ** -0.5)


@pytest.mark.parametrize("t,group", [(20, 1), (33, 2)])
def test_most_kv_heads(tq, signs, t, group):
    """65535 KV heads, the most the library takes: the per-lane record
    offsets within a piece reach 255 tokens' stride apart only through the
    head count, and one chunk per head gives 65535 blocks. Sampled KV heads
    (the first, the last and some between) are checked, each against the
    oracle on its own records alone."""
    hkv = 65535
    rec = datagen.decode_records(2 * t * hkv, seed=40 + t).numpy()
    k, v = rec[: t * hkv], rec[t * hkv:]
    q = np.random.default_rng(t).standard_normal((group * hkv, 128)).astype(np.float32) * 0.05
    got, qq = run(tq, q, k, v, hkv, signs, 128 ** -0.5)
    kt, vt = k.reshape(t, hkv, 56), v.reshape(t, hkv, 56)
    for j in (0, 1, 4097, 32768, 54321, hkv - 2, hkv - 1):
        h = slice(j * group, (j + 1) * group)
        compare(got[h], qq[h], np.ascontiguousarray(kt[:, j]), np.ascontiguousarray(vt[:, j]), 1,
                signs, 128 ** -0.5)


def test_random_records_large(tq, signs):
    """Uniform random index bytes with norms and scales as in the decode
    workload, 4096 tokens x 4 KV heads, 8 query heads per KV head."""
    rec = datagen.decode_records(2 * 4096 * 4, seed=8).numpy()
    q = np.random.default_rng(9).standard_normal((32, 128)).astype(np.float32) * 0.05
    check(tq, q, rec[: 4096 * 4], rec[4096 * 4:], 4, signs, 128 ** -0.5)


def test_closed_forms(tq, signs):
    hkv, hq = 2, 4
    # one token: the output is the value vector
    k, v = gaussian_records(hkv, 11, signs), gaussian_records(hkv, 12, signs)
    q = np.random.default_rng(13).standard_normal((hq, 128)).astype(np.float32)
    out = tq.tq3_decode_attention(torch.from_numpy(q).to(DEV), torch.from_numpy(k).to(DEV),
                                  torch.from_numpy(v).to(DEV), hkv, signs).cpu().numpy()
    vd = oracle.tq3_dequantize(v, signs)
    for h in range(hq):
        assert np.allclose(out[h], vd[h // 2], rtol=0, atol=2e-6 * np.abs(vd[h // 2]).max())
    # zero scale: the mean value
    t = 77
    k, v = gaussian_records(t * hkv, 14, signs), gaussian_records(t * hkv, 15, signs)
    out = tq.tq3_decode_attention(torch.from_numpy(q).to(DEV), torch.from_numpy(k).to(DEV),
                                  torch.from_numpy(v).to(DEV), hkv, signs, 0.0).cpu().numpy()
    vd = oracle.tq3_dequantize(v, signs).astype(np.float64).reshape(t, hkv, 128)
    for h in range(hq):
        assert np.allclose(out[h], vd[:, h // 2].mean(0), rtol=0,
                           atol=1e-5 * np.abs(vd[:, h // 2]).max())


def test_argument_errors(tq, signs):
    q = torch.zeros(12, 128, device=DEV)
    rec = torch.zeros(8, 56, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        tq.tq3_decode_attention(q, rec, rec, 8, signs)  # 12 heads over 8
    with pytest.raises(ValueError):
        tq.tq3_decode_attention(q[:8], rec, rec[:4], 8, signs)
    with pytest.raises(ValueError):
        tq.tq3_decode_attention(torch.zeros(24, 128, device=DEV), rec, rec, 8, signs)  # group 3


def test_workspace_reuse(tq, signs):
    """One workspace serves consecutive calls of different sizes."""
    hkv, hq = 4, 16
    big = tq.tq3_attention_workspace_bytes(3000, hq, hkv)
    ws = torch.empty(big, dtype=torch.uint8, device=DEV)
    for t, seed in ((3000, 30), (3000, 31), (700, 32), (3000, 33)):
        q = np.random.default_rng(seed).standard_normal((hq, 128)).astype(np.float32)
        k, v = gaussian_records(t * hkv, seed + 100, signs), gaussian_records(t * hkv, seed + 200, signs)
        out = tq.tq3_decode_attention(torch.from_numpy(q).to(DEV), torch.from_numpy(k).to(DEV),
                                      torch.from_numpy(v).to(DEV), hkv, signs, 0.1, workspace=ws)
        ref = oatt.tq3_decode_attention(q, k, v, hkv, signs, 0.1)
        vmax = np.abs(oracle.tq3_dequantize(v, signs)).max()
        assert np.abs(out.cpu().numpy() - ref).max() <= 2e-5 * vmax
