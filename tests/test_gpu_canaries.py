"""Canary bytes around every output buffer of the library.

Each output is a view into a larger buffer whose 256 bytes before and after
it are filled with a pattern; after the call (and a device synchronization)
the guards must be unchanged. Sizes are ragged and span the launch paths of
each entry point (small, one-tile and many-tile launches; OrbitQuant rows of
96, 3072 and 12288; the linear layer's few-rows, small-tile, square-tile and
tall-tile kernels). The values themselves are checked against the oracle in
the other GPU tests; here a kernel writing past either end of its output is
caught.
"""
import numpy as np
import pytest
import torch

import datagen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GUARD_BYTES = 256
PATTERN = 0xA5


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import randomized_hadamard_lloyd_amd as m
    return m


class Guarded:
    """A contiguous `shape` tensor of `dtype` inside a pattern-filled buffer."""

    def __init__(self, shape, dtype):
        es = torch.empty((), dtype=dtype).element_size()
        numel = int(np.prod(shape)) if len(shape) else 1
        body = numel * es
        self.raw = torch.full((GUARD_BYTES + body + GUARD_BYTES,), PATTERN, dtype=torch.uint8,
                              device=DEV)
        self.body = body
        self.t = self.raw[GUARD_BYTES:GUARD_BYTES + body].view(dtype).view(shape)

    def check(self, what):
        torch.cuda.synchronize()
        head = self.raw[:GUARD_BYTES]
        tail = self.raw[GUARD_BYTES + self.body:]
        assert bool((head == PATTERN).all()), f"{what}: bytes before the output overwritten"
        assert bool((tail == PATTERN).all()), f"{what}: bytes after the output overwritten"


@pytest.mark.parametrize("n", [1, 17, 1000, 4097])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_tq3_outputs(tq, n, dtype):
    signs = datagen.tq3_signs()
    x = datagen.gaussian_vectors(n, seed=n).to(dtype).to(DEV)
    rec = Guarded((n, 1, 56), torch.uint8)
    tq.tq3_quantize(x, signs, out=rec.t)
    rec.check("tq3_quantize")
    for odt in (torch.float32, torch.bfloat16, torch.float16):
        y = Guarded((n, 128), odt)
        tq.tq3_dequantize(rec.t, signs, dtype=odt, out=y.t)
        y.check(f"tq3_dequantize {odt}")
    p, nr, sc = Guarded((n, 1, 48), torch.uint8), Guarded((n, 1), torch.float32), \
        Guarded((n, 1), torch.float32)
    tq.tq3_quantize_split(x, signs, packed=p.t, norms=nr.t, scales=sc.t)
    for g, nm in ((p, "packed"), (nr, "norms"), (sc, "scales")):
        g.check(f"tq3_quantize_split {nm}")
    y = Guarded((n, 128), dtype)
    tq.tq3_dequantize_split(p.t, nr.t, sc.t, signs, dtype=dtype, out=y.t)
    y.check("tq3_dequantize_split")


@pytest.mark.parametrize("d,rows", [(96, 1), (96, 37), (3072, 37), (12288, 5)])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_orbit_codec_outputs(tq, d, rows, bits):
    perm, sg = datagen.rpbh_params(d)
    cb = tq.orbit_make_codebook(bits, d)
    w = datagen.orbit_weight(rows=rows, d=d, seed=d + rows).to(DEV)
    packed = Guarded((rows, d * bits // 8), torch.uint8)
    norms = Guarded((rows,), torch.float32)
    tq.orbit_quantize_weight(w, bits, perm.to(DEV), sg.to(DEV), cb, packed=packed.t,
                             row_norms=norms.t)
    packed.check("orbit_quantize_weight packed")
    norms.check("orbit_quantize_weight row_norms")
    inv = torch.argsort(perm).to(DEV)
    for rotated in (True, False):
        for odt in (torch.float32, torch.bfloat16):
            out = Guarded((rows, d), odt)
            tq.orbit_dequantize(packed.t, norms.t, d, bits, inv, sg.to(DEV), cb,
                                rotated_only=rotated, dtype=odt, out=out.t)
            out.check(f"orbit_dequantize rotated={rotated} {odt}")


@pytest.mark.parametrize("d,rows", [(96, 1), (3072, 37), (12288, 3)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_orbit_rotate_outputs(tq, d, rows, dtype):
    perm, sg = datagen.rpbh_params(d)
    x = torch.randn(rows, d, generator=torch.Generator().manual_seed(d)).to(dtype).to(DEV)
    out = Guarded((rows, d), dtype)
    tq.orbit_rotate(x, perm.to(DEV), sg.to(DEV), out=out.t)
    out.check("orbit_rotate")


@pytest.mark.parametrize("m", [1, 17, 40, 64, 100, 300])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d_in,d_out,bits", [(96, 65, 3), (1024, 300, 4), (32, 130, 2)])
def test_orbit_linear_outputs(tq, m, dtype, d_in, d_out, bits):
    g = torch.Generator().manual_seed(m + d_in)
    packed = torch.randint(0, 256, (d_out, d_in * bits // 8), generator=g,
                           dtype=torch.uint8).to(DEV)
    norms = (torch.rand(d_out, generator=g) + 0.5).to(DEV)
    cb = tq.orbit_make_codebook(bits, d_in)
    x = torch.randn(m, d_in, generator=g).to(dtype).to(DEV)
    bias = torch.randn(d_out, generator=g).to(dtype).to(DEV)
    y = Guarded((m, d_out), dtype)
    tq.orbit_linear(x, packed, norms, bits, cb, bias=bias, out=y.t)
    y.check(f"orbit_linear m={m}")


@pytest.mark.parametrize("n_tok,hkv,group", [(1, 1, 1), (300, 2, 4), (4097, 8, 8)])
def test_attention_outputs(tq, n_tok, hkv, group):
    signs = datagen.tq3_signs()
    g = torch.Generator().manual_seed(n_tok)
    k = tq.tq3_quantize(torch.randn(n_tok * hkv, 128, generator=g).to(DEV), signs)
    v = tq.tq3_quantize(torch.randn(n_tok * hkv, 128, generator=g).to(DEV), signs)
    hq = hkv * group
    q = torch.randn(hq, 128, generator=g).to(DEV)
    ws = Guarded((tq.tq3_attention_workspace_bytes(n_tok, hq, hkv),), torch.uint8)
    for odt in (torch.float32, torch.bfloat16):
        out = Guarded((hq, 128), odt)
        tq.tq3_decode_attention(q, k, v, hkv, signs, dtype=odt, workspace=ws.t, out=out.t)
        out.check("tq3_decode_attention out")
        ws.check("tq3_decode_attention workspace")
        out2 = Guarded((hq, 128), odt)
        tq.tq3_decode_attention_noalloc(q, k, v, hkv, signs, dtype=odt, out=out2.t)
        out2.check("tq3_decode_attention_noalloc out")


@pytest.mark.parametrize("m,d,n", [(1, 64, 40), (17, 96, 65), (300, 3072, 130), (33, 4096, 64)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_orbit_tiled_outputs(tq, m, d, n, dtype):
    perm, sg = datagen.rpbh_params(d)
    x = torch.randn(m, d, generator=torch.Generator().manual_seed(m + d)).to(dtype).to(DEV)
    xt = Guarded((tq.orbit_tiled_bytes(m, d) // 2,), dtype)
    tq.orbit_rotate_tiled(x, perm.to(DEV), sg.to(DEV), out=xt.t)
    xt.check("orbit_rotate_tiled")
    bits = 3
    g = torch.Generator().manual_seed(n)
    packed = torch.randint(0, 256, (n, d * bits // 8), generator=g, dtype=torch.uint8).to(DEV)
    norms = (torch.rand(n, generator=g) + 0.5).to(DEV)
    y = Guarded((m, n), dtype)
    tq.orbit_linear_tiled(xt.t, m, packed, norms, bits, tq.orbit_make_codebook(bits, d),
                          out=y.t)
    y.check("orbit_linear_tiled")
