"""GPU parity of the TQ3 kernels' software-pipelined instantiations.

The launchers switch to a pipelined loop (the next vector's loads issued before
the current vector is processed) once every wave runs at least 16 grid-stride
iterations: with G resident blocks (occupancy x 256 compute units) that is
n_vec >= 16 * 64 * G, about 2^20 vectors at 4 blocks per CU and 2^21 at 8.
These tests run every pipelined instantiation at 2^21 vectors, above the
switch for any occupancy, plus the structured workload's full 2^20 records,
and compare every record and every reconstructed row with the oracle.

Source: "ComfyUI-TurboQuant: tq3_core.py", tq3_quantize / tq3_dequantize
(record and three-array forms).
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from parity_util import compare_reconstruction, compare_tq3_records, split_records

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
N_PIPE = 1 << 21
CHUNK = 1 << 17


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import randomized_hadamard_lloyd_amd as m
    return m


@pytest.fixture(scope="module")
def signs():
    return datagen.tq3_signs()


def assert_records(g, x32, signs):
    o = oracle.tq3_quantize(x32, signs)
    if not np.array_equal(g, o):
        for a in range(0, o.shape[0], CHUNK):
            st = compare_tq3_records(g[a:a + CHUNK], o[a:a + CHUNK],
                                     oracle.tq3_scaled_coeffs(x32[a:a + CHUNK], signs))
            assert st["exact"], (a, st)
    return o


def assert_rows(y, rec, signs, dtype):
    """Every reconstructed row equals the oracle's (RNE-narrowed for bf16/fp16)."""
    y = y.reshape(-1, 128).cpu()
    for a in range(0, rec.shape[0], CHUNK):
        part = rec[a:a + CHUNK]
        o = oracle.tq3_dequantize(part, signs)
        ref = torch.from_numpy(o).to(dtype)
        if not torch.equal(y[a:a + CHUNK], ref):
            _, norms, _ = split_records(part)
            st = compare_reconstruction(y[a:a + CHUNK], o, norms, dtype)
            assert st["exact"], (a, st)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
def test_pipelined_quantize(tq, signs, dtype):
    """2^21 vectors of the KV-cache shape ([262144 tokens, 8 heads, 128])."""
    x = datagen.kv_cache("K", tokens=N_PIPE // 8, dtype=dtype)
    print(f"quantize {dtype} n={N_PIPE}", flush=True)
    rec = tq.tq3_quantize(x.to(DEV), signs)
    torch.cuda.synchronize()
    g = rec.cpu().numpy().reshape(-1, 56)
    assert_records(g, x.to(torch.float32).reshape(-1, 128).numpy(), signs)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_pipelined_dequantize(tq, signs, dtype):
    """2^21 random records (the decode workload's recipe) to each output type."""
    rec = datagen.decode_records(N_PIPE, seed=41)
    print(f"dequantize {dtype} n={N_PIPE}", flush=True)
    y = tq.tq3_dequantize(rec.to(DEV), signs, dtype=dtype)
    torch.cuda.synchronize()
    assert_rows(y, rec.numpy(), signs, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
def test_structured_full_dequantize(tq, signs, dtype):
    """The structured workload's 2^20 records (the oracle's quantization of all
    four quarters), every row dequantized on the GPU and compared."""
    x = datagen.structured_blocks()
    rec = oracle.tq3_quantize(x.numpy(), signs)
    print(f"structured dequantize {dtype} n={rec.shape[0]}", flush=True)
    y = tq.tq3_dequantize(torch.from_numpy(rec).to(DEV), signs, dtype=dtype)
    torch.cuda.synchronize()
    assert_rows(y, rec, signs, dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_pipelined_split_layout(tq, signs, dtype):
    """tq3_quantize_split / tq3_dequantize_split at 2^21 vectors."""
    x = datagen.kv_cache("V", tokens=N_PIPE // 8, dtype=dtype)
    print(f"split {dtype} n={N_PIPE}", flush=True)
    packed, norms, scales = tq.tq3_quantize_split(x.to(DEV), signs)
    y = tq.tq3_dequantize_split(packed, norms, scales, signs, dtype=dtype)
    torch.cuda.synchronize()
    g = np.concatenate([packed.cpu().numpy().reshape(-1, 48),
                        norms.cpu().numpy().reshape(-1, 1).view(np.uint8),
                        scales.cpu().numpy().reshape(-1, 1).view(np.uint8)], axis=1)
    o = assert_records(g, x.to(torch.float32).reshape(-1, 128).numpy(), signs)
    assert_rows(y, o, signs, dtype)
