"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module holds no codec arithmetic: it only draws random numbers with torch's
CPU generator and shapes them like the workloads the codec pages describe.
Random numbers that the methods themselves draw (the TQ3 sign vector, the
RPBH permutation and signs) are produced here and passed to both the oracle
and the GPU library as inputs.

Workloads (sizes are the full ones; every builder takes a smaller count for
parity tests):
  1. Gaussian round trip: 4096 x 128 fp32 ~ N(0, 1), seed 0.
  2. KV-cache layer: K and V, [32768 tokens, 8 heads, 128] bf16. z ~ N(0,1);
     four channel indices (drawn once, shared by heads, tokens and both
     tensors) multiplied by 20; each token's 8x128 values multiplied by
     exp(N(0, 0.5^2)); rounded to bf16. Seeds 2 (K) and 3 (V); the channel
     draw uses seed 1.
  3. Structured blocks: 2^20 fp32 vectors in four contiguous quarters --
     constants ~ U(-3, 3); cos(2 pi f t / 128 + phase), f in {1,2,3},
     phase ~ U(0, 2 pi); N(0, 0.01^2) with one uniformly chosen coordinate
     set to 10; N(0, 1). Seed 3.
  4. Decode records: 2^24 records of 56 bytes: 48 uniform random bytes, an
     fp32 norm ~ U(0.5, 20), an fp32 scale ~ U(0.5, 3). Seed 4.
  5. OrbitQuant weight: [12288, 3072] fp32 ~ N(0, 0.02^2), seed 5.
"""
import math

import torch

TQ3_SIGN_SEED = 42
RPBH_SEED_BASE = 0x0EB17

KV_TOKENS = 32768
KV_HEADS = 8
HEAD_DIM = 128


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


# ---------------------------------------------- draws the methods make ---

def tq3_signs(seed: int = TQ3_SIGN_SEED, dim: int = 128) -> torch.Tensor:
    """The TQ3 page's deterministic sign vector: a CPU generator seeded with
    `seed`, `dim` fair 0/1 draws as float32, mapped to -1/+1."""
    bits = torch.randint(0, 2, (dim,), generator=_gen(seed), dtype=torch.float32)
    return bits * 2.0 - 1.0


def rpbh_params(d: int):
    """The OrbitQuant page's rotation draw for input dimension d: a generator
    seeded with 0x0EB17 + d gives randperm(d) (int64), then d fair 0/1 draws
    as int8 mapped to -1/+1, in that order from the same generator."""
    g = _gen(RPBH_SEED_BASE + d)
    perm = torch.randperm(d, generator=g)
    signs = torch.randint(0, 2, (d,), generator=g, dtype=torch.int8) * 2 - 1
    return perm, signs


# --------------------------------------------------------- workloads ---

def gaussian_vectors(n: int = 4096, seed: int = 0) -> torch.Tensor:
    """Workload 1: n x 128 fp32 standard normal."""
    return torch.randn(n, HEAD_DIM, generator=_gen(seed), dtype=torch.float32)


def kv_outlier_channels(seed: int = 1, count: int = 4) -> torch.Tensor:
    """The four outlier channel indices of workload 2 (distinct, in [0,128))."""
    return torch.randperm(HEAD_DIM, generator=_gen(seed))[:count].sort().values


def kv_cache(which: str = "K", tokens: int = KV_TOKENS, heads: int = KV_HEADS,
             dtype=torch.bfloat16) -> torch.Tensor:
    """Workload 2: one layer's K or V, [tokens, heads, 128] (token-major)."""
    seed = {"K": 2, "V": 3}[which]
    g = _gen(seed)
    z = torch.randn(tokens, heads, HEAD_DIM, generator=g, dtype=torch.float32)
    z[:, :, kv_outlier_channels()] *= 20.0
    tok = torch.exp(torch.randn(tokens, 1, 1, generator=g) * 0.5)
    return (z * tok).to(dtype)


def structured_blocks(n: int = 1 << 20, seed: int = 3) -> torch.Tensor:
    """Workload 3: n fp32 vectors (n divisible by 4) in four quarters."""
    assert n % 4 == 0
    q = n // 4
    g = _gen(seed)
    const = (torch.rand(q, 1, generator=g) * 6.0 - 3.0).expand(q, HEAD_DIM)
    t = torch.arange(HEAD_DIM, dtype=torch.float32)
    freq = torch.randint(1, 4, (q, 1), generator=g).to(torch.float32)
    phase = torch.rand(q, 1, generator=g) * (2.0 * math.pi)
    cosines = torch.cos(2.0 * math.pi * freq * t / HEAD_DIM + phase)
    spikes = torch.randn(q, HEAD_DIM, generator=g) * 0.01
    where = torch.randint(0, HEAD_DIM, (q,), generator=g)
    spikes[torch.arange(q), where] = 10.0
    normal = torch.randn(q, HEAD_DIM, generator=g)
    return torch.cat([const, cosines, spikes, normal]).contiguous().to(torch.float32)


def decode_records(n: int = 1 << 24, seed: int = 4) -> torch.Tensor:
    """Workload 4: uint8 [n, 56] records with uniform random index bytes."""
    g = _gen(seed)
    rec = torch.empty(n, 56, dtype=torch.uint8)
    rec[:, :48] = torch.randint(0, 256, (n, 48), generator=g, dtype=torch.uint8)
    norms = torch.rand(n, generator=g) * 19.5 + 0.5
    scales = torch.rand(n, generator=g) * 2.5 + 0.5
    rec[:, 48:52] = norms.view(torch.uint8).view(n, 4)
    rec[:, 52:56] = scales.view(torch.uint8).view(n, 4)
    return rec


def orbit_weight(rows: int = 12288, d: int = 3072, seed: int = 5) -> torch.Tensor:
    """Workload 5: fp32 weight [rows, d] ~ N(0, 0.02^2)."""
    return torch.randn(rows, d, generator=_gen(seed), dtype=torch.float32) * 0.02


def attention_queries(n_heads: int = 32, seed: int = 6) -> torch.Tensor:
    """Decode-step queries for attention over the KV layer: [n_heads, 128]
    fp32 N(0, 1) (32 query heads over the layer's 8 KV heads)."""
    return torch.randn(n_heads, HEAD_DIM, generator=_gen(seed), dtype=torch.float32)


def sign_mask_bytes(signs) -> bytes:
    """16-byte little-endian mask of a 128-entry sign vector: bit j set means
    sign j is negative. (Pure reformatting of a drawn input.)"""
    m = 0
    for j, s in enumerate(torch.as_tensor(signs).reshape(-1).tolist()):
        if s < 0:
            m |= 1 << j
    return m.to_bytes(16, "little")
