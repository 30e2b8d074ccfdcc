"""Pins of the oracle's bit packing.

Sources: "ComfyUI-TurboQuant: tq3_core.py", _pack_3bit/_unpack_3bit (groups
of eight 3-bit indices form a 24-bit word stored as three little-endian
bytes; 48 bytes per 128 indices) and the 56-byte record of its docstring;
"orbit_quant.py", pack_codes/unpack_codes (flat bit-matrix, most significant
bit first, zero padding to a whole byte).
"""
import numpy as np
import pytest


def page_group_pack_3bit(idx):
    """The TQ3 page's formulation: per group g of 8 values, word = OR of
    v_i << 3i, bytes 3g..3g+2 = word's bytes, low byte first."""
    idx = np.asarray(idx, dtype=np.int64).reshape(-1, 128)
    out = np.zeros((idx.shape[0], 48), dtype=np.uint8)
    for g in range(16):
        word = np.zeros(idx.shape[0], dtype=np.int64)
        for i in range(8):
            word |= idx[:, 8 * g + i] << (3 * i)
        out[:, 3 * g] = word & 0xFF
        out[:, 3 * g + 1] = (word >> 8) & 0xFF
        out[:, 3 * g + 2] = (word >> 16) & 0xFF
    return out


def page_bitmatrix_pack_msb(codes, bits):
    """The OrbitQuant page's formulation: expand each code to a row of bits
    (most significant first), regroup the flat bit list in eights, weight by
    128, 64, ..., 1."""
    flat = np.asarray(codes, dtype=np.uint8).reshape(-1)
    pad = (-flat.size) % 8
    flat = np.concatenate([flat, np.zeros(pad, dtype=np.uint8)])
    shifts = np.arange(bits - 1, -1, -1, dtype=np.uint8)
    bitmat = (flat[:, None] >> shifts) & 1
    bytemat = bitmat.reshape(-1, 8).astype(np.int64)
    weights = np.array([1 << i for i in range(7, -1, -1)], dtype=np.int64)
    return (bytemat * weights).sum(-1).astype(np.uint8)


def test_tq3_group_pack_equals_lsb_stream(oracle_mod):
    rng = np.random.default_rng(3)
    idx = rng.integers(0, 8, size=(64, 128), dtype=np.uint8)
    want = page_group_pack_3bit(idx)
    got = np.stack([oracle_mod.pack(r, 3) for r in idx])
    assert got.shape == (64, 48)
    assert np.array_equal(got, want)


def test_tq3_pack_round_trip(oracle_mod):
    # the TQ3 page's self-test [3]: unpack(pack(i)) == i for random (16,128)
    rng = np.random.default_rng(5)
    idx = rng.integers(0, 8, size=(16, 128), dtype=np.uint8)
    for r in idx:
        assert np.array_equal(oracle_mod.unpack(oracle_mod.pack(r, 3), 128, 3), r)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("msb", [False, True])
def test_exhaustive_value_position(oracle_mod, bits, msb):
    # every value at every position of a 64-code stream, others zero
    for pos in range(64):
        for v in range(1 << bits):
            codes = np.zeros(64, dtype=np.uint8)
            codes[pos] = v
            packed = oracle_mod.pack(codes, bits, msb_first=msb)
            assert packed.size == 64 * bits // 8
            assert np.array_equal(oracle_mod.unpack(packed, 64, bits, msb_first=msb), codes)
            # the value's bits sit exactly at stream bits bits*pos .. bits*pos+bits-1
            stream = np.unpackbits(packed, bitorder="big" if msb else "little")
            ones = set(np.nonzero(stream)[0].tolist())
            if msb:
                want = {bits * pos + t for t in range(bits) if (v >> (bits - 1 - t)) & 1}
            else:
                want = {bits * pos + t for t in range(bits) if (v >> t) & 1}
            assert ones == want


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_msb_pack_equals_page_bitmatrix(oracle_mod, bits):
    # counts are multiples of 8: the page pads the code count to a multiple of
    # 8 before packing, which only differs from ceil(count*bits/8) bytes
    # otherwise, and weight rows always hold a multiple of 32 codes
    rng = np.random.default_rng(bits)
    for count in (8, 96, 3072, 3080):
        codes = rng.integers(0, 1 << bits, size=count, dtype=np.uint8)
        assert np.array_equal(oracle_mod.pack(codes, bits, msb_first=True),
                              page_bitmatrix_pack_msb(codes, bits))


def test_record_is_56_bytes(oracle_mod):
    # 128 * 3 bits = 48 bytes, plus fp32 norm and fp32 scale
    x = np.random.default_rng(0).standard_normal((3, 128)).astype(np.float32)
    signs = np.ones(128, dtype=np.float32)
    rec = oracle_mod.tq3_quantize(x, signs)
    assert rec.shape == (3, 56)
    assert 128 * 3 // 8 + 4 + 4 == 56
