"""The C-ABI library loads and exports every symbol include/tq.h declares, and its
host-side helpers agree with the oracle (no GPU needed)."""
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "randomized_hadamard_lloyd_amd", "libtq.so")


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "tq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def tq():
    if not os.path.exists(LIB):
        pytest.skip("libtq.so not built")
    import randomized_hadamard_lloyd_amd as m
    return m


def test_exports_every_declared_symbol(tq):
    names = declared_symbols()
    assert {"tq3_quantize", "tq3_dequantize", "orbit_quantize_weight", "orbit_dequantize"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(tq.EXPORTS) == set(names)


def test_host_helpers(tq):
    assert tq.tq3_record_bytes() == 56
    assert tq.orbit_block_size(3072) == 1024
    assert tq.orbit_block_size(4096) == 4096
    assert tq.orbit_block_size(0) == 0
    comp, orig, ratio = tq.tq3_memory_bytes((2, 64, 64, 2048, 128))
    assert (comp, orig) == (939_524_096, 4_294_967_296) and ratio > 4.0


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_codebook_matches_oracle(tq, bits):
    import oracle
    assert np.array_equal(tq.orbit_make_codebook(bits, 3072).numpy(),
                          oracle.orbit_codebook(bits, 3072))
    assert np.array_equal(tq.orbit_make_codebook(bits, 96).numpy(), oracle.orbit_codebook(bits, 96))
    lm = tq.tq_gaussian_lloyd_max(bits).numpy()
    assert np.array_equal(lm.astype(np.float32), oracle.gaussian_lloyd_max(bits))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_codebook_matches_oracle_every_width(tq, bits):
    """The product's host codebook equals the oracle's at every input width the
    GPU tests use: each multiple of 32 up to 16384 and a few wider ones."""
    import oracle
    widths = list(range(32, 16385, 32)) + [20480, 24576, 28672, 32768, 65536]
    for d in widths:
        assert np.array_equal(tq.orbit_make_codebook(bits, d).numpy(),
                              oracle.orbit_codebook(bits, d)), d


def test_sign_mask_matches_golden(tq):
    import json
    import datagen
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "tq3_signs.json")))
    m = tq.sign_mask(datagen.tq3_signs())
    assert hex(int.from_bytes(m, "little")) == g["mask_hex"]


def test_argument_errors_without_gpu(tq):
    L = tq.lib
    # argument checks run before any device call
    assert L.tq3_quantize(None, 9, 4, 128, None, None, None) == 3
    assert L.tq3_quantize(None, 0, 4, 100, None, None, None) == 2
    assert L.tq3_quantize(None, 0, 0, 128, None, None, None) == 0
    assert L.tq3_quantize_split(None, 9, 4, 128, None, None, None, None, None) == 3
    assert L.tq3_quantize_split(None, 0, 4, 136, None, None, None, None, None) == 1
    assert L.tq3_quantize_split(None, 0, 0, 128, None, None, None, None, None) == 0
    assert L.tq3_dequantize_split(None, None, None, 4, None, None, 0, 64, None) == 2
    assert L.tq3_dequantize_split(None, None, None, -1, None, None, 0, 128, None) == 2
    assert L.tq3_dequantize_split(None, None, None, 4, None, None, 1, 128, None) == 1
    cb = tq._host_f32([-1.0, -0.5, 0.5, 1.0])
    import ctypes
    p = ctypes.cast(cb, ctypes.c_void_p)
    assert L.orbit_quantize_weight(None, 4, 3072, 5, None, None, p, 0, None, None, None) == 4
    assert L.orbit_quantize_weight(None, 4, 48, 2, None, None, p, 0, None, None, None) == 5
    assert L.orbit_quantize_weight(None, 4, 3072, 2, None, None, p, 3, None, None, None) == 8
    assert L.orbit_quantize_weight(None, 0, 3072, 2, None, None, p, 0, None, None, None) == 0
    assert L.orbit_quantize_weight(None, 4, 3072, 2, None, None, p, 0, None, None, None) == 1
    bad = tq._host_f32([1.0, -0.5, 0.5, 1.0])
    assert L.orbit_quantize_weight(None, 4, 3072, 2, None, None,
                                   ctypes.cast(bad, ctypes.c_void_p), 0, None, None, None) == 8
    assert L.orbit_dequantize(None, None, 4, 3072, 2, None, None, p, 0, 0, None, 7, None) == 3
    assert tq.lib.tq_status_str(5).decode().startswith("Hadamard")


def test_attention_arguments_without_gpu(tq):
    L = tq.lib
    assert tq.tq3_attention_workspace_bytes(0, 8, 8) == 0
    assert tq.tq3_attention_workspace_bytes(10, 12, 8) == 0   # 12 query heads over 8
    assert tq.tq3_attention_workspace_bytes(10, 24, 8) == 0   # group of 3
    assert tq.tq3_attention_workspace_bytes(10, 8, 0) == 0
    assert tq.tq3_attention_workspace_bytes(10, 65536, 65536) == 0   # > 65535 KV heads
    assert tq.tq3_attention_workspace_bytes(10, 65535, 65535) > 0
    assert tq.tq3_attention_workspace_bytes((1 << 28) + 1, 8, 8) == 0   # tokens x heads > 2^31
    assert tq.tq3_attention_workspace_bytes(1 << 28, 8, 8) > 0
    ws = tq.tq3_attention_workspace_bytes(32768, 32, 8)
    assert ws > 0 and ws % 16 == 0
    assert tq.tq3_attention_workspace_bytes(1, 8, 1) > 0
    m = bytes(16)
    args = lambda **kw: dict(dict(q=1 << 20, qd=0, hq=32, k=1 << 20, v=1 << 20, t=32768, hkv=8,
                                  m=m, sc=0.088, ws=1 << 20, wsb=ws, o=1 << 20, od=0), **kw)
    call = lambda a: L.tq3_decode_attention(a["q"], a["qd"], a["hq"], a["k"], a["v"], a["t"],
                                            a["hkv"], a["m"], a["sc"], a["ws"], a["wsb"], a["o"],
                                            a["od"], None)
    assert call(args(qd=7)) == 3
    assert call(args(od=7)) == 3
    assert call(args(t=0)) == 2
    assert call(args(hq=24)) == 2
    assert call(args(sc=float("nan"))) == 8
    assert call(args(q=None)) == 1
    assert call(args(wsb=ws - 1)) == 8
    assert call(args(q=(1 << 20) + 4)) == 6
    assert call(args(k=(1 << 20) + 4)) == 6


def test_caller_buffers_are_validated_before_any_call(tq):
    """The C entry points cannot see the size or type of a buffer, so the binding
    rejects a caller-given output that is not exactly what the kernels write
    (these checks run before the GPU check, so CPU tensors exercise them)."""
    import torch
    x = torch.zeros(3, 256)
    signs = torch.ones(128)
    with pytest.raises(ValueError, match="out must be"):
        tq.tq3_quantize(x, signs, out=torch.empty(6 * 56 - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="out must be"):
        tq.tq3_quantize(x, signs, out=torch.empty(6 * 56, dtype=torch.int8))
    with pytest.raises(ValueError, match="out must be"):
        tq.tq3_quantize(x, signs, out=torch.empty(6 * 112, dtype=torch.uint8)[::2])
    rec = torch.zeros(5, 56, dtype=torch.uint8)
    # an fp32 result into a bf16 buffer would write twice the buffer's bytes
    with pytest.raises(ValueError, match="out must be"):
        tq.tq3_dequantize(rec, signs, out=torch.empty(5 * 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out must be"):
        tq.tq3_dequantize(rec, signs, dtype=torch.bfloat16,
                          out=torch.empty(5 * 128 - 8, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out must be"):
        tq.tq3_dequantize_split(torch.zeros(5, 48, dtype=torch.uint8), torch.zeros(5),
                                torch.zeros(5), signs, out=torch.empty(5 * 128,
                                                                       dtype=torch.float16))
    with pytest.raises(ValueError, match="out must be"):
        tq.tq3_decode_attention(torch.zeros(4, 128), torch.zeros(8, 56, dtype=torch.uint8),
                                torch.zeros(8, 56, dtype=torch.uint8), 2, signs,
                                out=torch.empty(4, 127))
    with pytest.raises(ValueError, match="workspace"):
        tq.tq3_decode_attention(torch.zeros(4, 128), torch.zeros(8, 56, dtype=torch.uint8),
                                torch.zeros(8, 56, dtype=torch.uint8), 2, signs,
                                workspace=torch.empty(4096, dtype=torch.uint8)[::2])


def test_orbit_dequantize_arguments_are_validated(tq):
    import torch
    d, bits, rows = 256, 3, 4
    packed = torch.zeros(rows, d * bits // 8, dtype=torch.uint8)
    norms = torch.ones(rows)
    inv, sg = torch.arange(d, dtype=torch.int32), torch.ones(d, dtype=torch.int8)
    cb = [float(v) for v in range(8)]
    with pytest.raises(ValueError, match="packed"):
        tq.orbit_dequantize(packed[:, :-1], norms, d, bits, inv, sg, cb)
    with pytest.raises(ValueError, match="codebook"):
        tq.orbit_dequantize(packed, norms, d, bits, inv, sg, cb[:4])
    with pytest.raises(ValueError, match="inv_perm"):
        tq.orbit_dequantize(packed, norms, d, bits, inv[:-1], sg, cb)
    with pytest.raises(ValueError, match="signs"):
        tq.orbit_dequantize(packed, norms, d, bits, inv, sg[:10], cb)
    with pytest.raises(ValueError, match="inv_perm"):
        tq.orbit_dequantize(packed, norms, d, bits, None, sg, cb)
    with pytest.raises(ValueError, match="out must be"):
        tq.orbit_dequantize(packed, norms, d, bits, inv, sg, cb, dtype=torch.float16,
                            out=torch.empty(rows, d))
    with pytest.raises(ValueError, match="bits"):
        tq.orbit_dequantize(packed, norms, d, 5, inv, sg, cb)


def test_tiled_forward_arguments_are_validated(tq):
    """orbit_rotate_tiled / orbit_linear_tiled reject bad arguments before any
    GPU call, and orbit_tiled_bytes follows the layout's padding rule."""
    import torch
    d = 96
    assert tq.orbit_tiled_bytes(1, d) == 16 * d * 2
    assert tq.orbit_tiled_bytes(16, d) == 16 * d * 2
    assert tq.orbit_tiled_bytes(17, d) == 32 * d * 2
    assert tq.orbit_tiled_bytes(4, 48) == 0 and tq.orbit_tiled_bytes(4, 32768) == 0
    assert tq.orbit_tiled_bytes(-1, d) == 0
    perm, sg = torch.arange(d, dtype=torch.int32), torch.ones(d, dtype=torch.int8)
    with pytest.raises(ValueError, match="bf16 or fp16"):
        tq.orbit_rotate_tiled(torch.zeros(4, d), perm, sg)
    with pytest.raises(ValueError, match="multiple of 32"):
        tq.orbit_rotate_tiled(torch.zeros(4, 48, dtype=torch.bfloat16), perm[:48], sg[:48])
    with pytest.raises(ValueError, match="out must be"):
        tq.orbit_rotate_tiled(torch.zeros(4, d, dtype=torch.bfloat16), perm, sg,
                              out=torch.empty(4 * d, dtype=torch.bfloat16))
    pk = torch.zeros(8 * d * 2 // 8, dtype=torch.uint8)
    nr = torch.ones(8)
    xt = torch.zeros(tq.orbit_tiled_bytes(4, d) // 2, dtype=torch.bfloat16)
    cb = [-1.0, -0.5, 0.5, 1.0]
    with pytest.raises(ValueError, match="bf16 or fp16"):
        tq.orbit_linear_tiled(xt.float(), 4, pk, nr, 2, cb)
    with pytest.raises(ValueError, match="tiled"):
        tq.orbit_linear_tiled(xt, 17, pk, nr, 2, cb)
    with pytest.raises(ValueError, match="packed"):
        tq.orbit_linear_tiled(xt, 4, pk[:-1], nr, 2, cb)
